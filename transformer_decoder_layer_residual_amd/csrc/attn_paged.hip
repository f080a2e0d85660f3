// attn_paged.hip -- paged grouped-query attention for q_len >= 1 new tokens
// per sequence (gfx950 MFMA).
//
// What it computes: sequence b brings q_len_b = cu_q[b+1] - cu_q[b] query
// tokens, which are the last q_len_b of its ctx_b = context_lens[b] cached
// positions; new token i sits at position p_i = ctx_b - q_len_b + i and
// attends over the cached positions 0 .. p_i of its kv head (ATB KV-cache
// page, section "speculative decoding": the paged attention verifies the
// candidate tokens of every sequence in one pass, with per-sequence query
// lengths and context lengths).  q_len 1 is the decode step, q_len = ctx a
// prefill that reads its keys from the cache, anything between a chunk of a
// prefill over a cached prefix.
//
// Design:
//   * a workgroup owns 128 query rows: QB = 128 / G tokens times the G query
//     heads that share kv head g, so each K/V byte it reads serves the whole
//     group;
//   * work items (sequence, query tile, key split) are numbered densely over
//     the sequences (wave prefix sum), one workgroup per (kv head, item); a
//     split covers CK consecutive positions (a multiple of 64 and of BS) and
//     its block ids are fetched into LDS once; positions after the tile's
//     last visible one are never read;
//   * K/V tiles of 64 keys go registers -> LDS (K row-major, V transposed),
//     the next tile's loads in flight while the current one is used; loads
//     are clamped into the split and masked when stored, so a NaN left in an
//     unwritten slot never reaches the arithmetic;
//   * S^T = K Q^T and O^T += V^T P^T on 16x16 MFMA fragments with one query
//     row per lane column, online softmax in registers (log2 domain); waves
//     whose rows are padding or see none of a tile skip its MFMAs;
//   * every (row, split) writes its unnormalised (o, m, l); a second kernel
//     merges the splits of each row in fixed order.
#include "attn_combine.hpp"
#include "dl_internal.hpp"

namespace dl {

namespace {

constexpr int kPgRows = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kPgBKV = 64;    // keys per tile
constexpr int kPgMaxSplitBlocks = 64;

__device__ __forceinline__ void scores_to_frag(Frag<bf16>& f, f32x4 a, f32x4 b) {
  f.v = bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
               (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}
__device__ __forceinline__ void scores_to_frag(Frag<float>& f, f32x4 a, f32x4 b) {
  f.lo = a;
  f.hi = b;
}
__device__ __forceinline__ void load_split_frag(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p0);
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(p1);
  f.v = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
__device__ __forceinline__ void load_split_frag(Frag<float>& f, const float* p0, const float* p1) {
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
}

// Per-sequence geometry shared by both kernels; every count is clamped to
// what the host sized the grid and the workspace for: the sequence's query
// rows to [0, Tq), its context to the table and to max_ctx.  cu_q ==
// nullptr: one new token per sequence (the decode step).
struct PgSeq {
  int q0, ql, ctx, first;  // first = position of new token 0
  __device__ PgSeq(const int32_t* cu_q, const int32_t* ctx_lens, int b, int Tq, int max_blocks,
                   int BS, int max_ctx) {
    q0 = cu_q ? min(max(cu_q[b], 0), Tq) : b;
    ql = cu_q ? max(min(cu_q[b + 1], Tq) - q0, 0) : 1;
    ctx = min(min(ctx_lens[b], max_blocks * BS), max_ctx);
    first = ctx - ql;
  }
};

// Splits that hold keys of the row at position p (keys 0 .. p).
__device__ __forceinline__ int row_splits(int p, int ck, int max_sp) {
  return p >= 0 ? min((p + ck) / ck, max_sp) : 0;
}

}  // namespace

constexpr int kPnKeys = 32;            // keys per wave step
constexpr int kPnMaxSplit = 8192;      // keys per split, at most
constexpr int kPnMaxSplitBlocks = kPnMaxSplit / 16;

// Keys per split for the narrow kernel: as large as keeps about one (uniform
// contexts, B <= 8) or two (ragged contexts) workgroups per CU over the
// estimated work (every sequence at max_ctx, or at half of it when ragged).
// Measured optimum on the 7B verification batch (4096), the 8B B64 decode
// (2048), 70B B4 x 4096 (512) and 70B B1 x 32768 (1024).
int narrow_split(int B, int Hkv, int max_ctx, int BS) {
  const int unit = BS > 128 ? BS : 128;
  const bool ragged = B > 8;
  const double work = (double)B * Hkv * max_ctx * (ragged ? 0.5 : 1.0);
  int ck = (int)(work / (256.0 * (ragged ? 2 : 1)));
  const int cap = (max_ctx + unit - 1) / unit * unit;
  if (ck > cap) ck = cap;
  ck = (ck + unit - 1) / unit * unit;
  const int lo = unit > 256 ? unit : 256;
  if (ck < lo) ck = lo;
  if (ck > kPnMaxSplit) ck = kPnMaxSplit / unit * unit;
  return ck;
}

PagedPlan plan_paged(int B, int Hq, int Hkv, int max_q_len, int max_context_len, int BS, int D,
                     int Tq) {
  PagedPlan pl{};
  const int G = Hq / Hkv;
  // at most 32 rows per kv head: the narrow kernel (one workgroup per CU,
  // splits of up to 8192 keys: its per-workgroup start and merge cost made
  // 1024-key splits 20% slower than 4096-key ones); else 128-row tiles
  pl.narrow = max_q_len * G <= 32 ? 1 : 0;
  pl.qb = (pl.narrow ? 32 : kPgRows) / G;
  pl.max_qt = max_q_len > 0 ? (max_q_len + pl.qb - 1) / pl.qb : 0;
  if (pl.narrow) {
    pl.ck = narrow_split(B, Hkv, max_context_len, BS);
  } else {
    // at least ~2048 workgroups at the longest context, splits of 256..1024 keys
    const int unit = BS > kPgBKV ? BS : kPgBKV;
    const long items = (long)B * Hkv * (pl.max_qt > 0 ? pl.max_qt : 1);
    const int want = (int)((2048 + items - 1) / items);
    int ck = (max_context_len + want - 1) / want;
    ck = (ck + unit - 1) / unit * unit;
    const int lo = unit > 256 ? unit : 256;
    if (ck < lo) ck = lo;
    if (ck > 1024) ck = 1024;
    pl.ck = ck;
  }
  pl.max_sp = max_context_len > 0 ? (max_context_len + pl.ck - 1) / pl.ck : 1;
  pl.ws_bytes = (size_t)Tq * Hq * pl.max_sp * (D + 2) * sizeof(float);
  return pl;
}

template <typename T, int D>
__global__ void __launch_bounds__(256, 2)
attn_paged_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
                  const int32_t* __restrict__ bt, int max_blocks, const int32_t* __restrict__ cu_q,
                  const int32_t* __restrict__ ctx_lens, int B, int Tq, int Hq, int Hkv, int BS,
                  float scale_log2, int ck, int max_qt, int max_sp, int max_ctx,
                  float* __restrict__ ws, int num_blocks, T* __restrict__ out) {
  constexpr int NT = 256, BKV = kPgBKV, VE = 16 / sizeof(T);
  constexpr int QS = 2, KTS = BKV / 16, DC = D / 32, DS = D / 16, KC = BKV / 32;
  constexpr int KLS = D + VE, VLS = BKV + VE;
  constexpr int K_IT = BKV * (D / VE) / NT, V_IT = (BKV / 2) * (D / VE) / NT;
  static_assert(K_IT * NT == BKV * (D / VE) && V_IT * NT == (BKV / 2) * (D / VE), "tile split");
  __shared__ __attribute__((aligned(16))) T Ks[2][BKV * KLS];
  __shared__ __attribute__((aligned(16))) T Vt[2][D * VLS];
  __shared__ int phys_s[kPgMaxSplitBlocks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int G = Hq / Hkv, QB = kPgRows / G;
  const int g = blockIdx.x % Hkv, item = blockIdx.x / Hkv;

  // ---- item -> (sequence, query tile, split)
  auto counts = [&](int bb, int& nqt, int& nsp) {
    const PgSeq s(cu_q, ctx_lens, bb, Tq, max_blocks, BS, max_ctx);
    nqt = s.ql > 0 ? min((s.ql + QB - 1) / QB, max_qt) : 0;
    nsp = s.ctx > 0 ? min((s.ctx + ck - 1) / ck, max_sp) : 0;
  };
  int b = -1, local = 0;
  for (int b0 = 0, base = 0; b0 < B; b0 += kWave) {
    int nqt = 0, nsp = 0;
    if (b0 + lane < B) counts(b0 + lane, nqt, nsp);
    const int n = nqt * nsp;
    int inc = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += y;
    }
    const int total = __shfl(inc, kWave - 1, kWave);
    if (item < base + total) {
      const bool mine = item >= base + inc - n && item < base + inc;
      const int L = __ffsll((unsigned long long)__ballot(mine)) - 1;
      b = b0 + L;
      local = item - base - __shfl(inc - n, L, kWave);
      break;
    }
    base += total;
  }
  if (b < 0) return;
  const PgSeq sq(cu_q, ctx_lens, b, Tq, max_blocks, BS, max_ctx);
  int nqt, nsp;
  counts(b, nqt, nsp);
  const int qt = local / nsp, sp = local % nsp;
  const int i_end = min(sq.ql, (qt + 1) * QB);  // tokens [qt*QB, i_end) of this tile
  const int kbeg = sp * ck;
  const int kend = min(min(sq.ctx, kbeg + ck), sq.first + i_end);
  if (kend <= kbeg) return;  // no row of the tile sees this split
  const int nt = (kend - kbeg + BKV - 1) / BKV;

  const int nb = (kend - kbeg + BS - 1) / BS;
  if (tid < nb) {
    const int p = bt[(int64_t)b * max_blocks + kbeg / BS + tid];
    phys_s[tid] = (p < 0 || p >= num_blocks) ? 0 : p;  // invalid ids read block 0
  }

  // ---- this lane's query rows: r = 32 * wave + 16 * qs + fr
  int tok[QS], head[QS];
  bool valid[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int r = 32 * wave + 16 * qs + fr;
    tok[qs] = qt * QB + r / G;
    head[qs] = g * G + r % G;
    valid[qs] = tok[qs] < sq.ql;
  }
  // the wave's last visible position (waves past the end of the tile see nothing)
  const int wave_tok_hi = qt * QB + (32 * wave + 31) / G;
  const bool wave_live = qt * QB + (32 * wave) / G < sq.ql;
  const int wave_lim = sq.first + min(wave_tok_hi, sq.ql - 1);

  Frag<T> qf[QS][DC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (valid[qs])
        qf[qs][dc].load(q + ((int64_t)(sq.q0 + tok[qs]) * Hq + head[qs]) * D + dc * 32 + 8 * fg);
      else
        qf[qs][dc].zero();
    }
  f32x4 o[DS][QS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) o[ds][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_i[QS], l_i[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    m_i[qs] = -INFINITY;
    l_i[qs] = 0.f;
  }

  __syncthreads();  // phys_s
  // ---- K/V tile loads: clamped into the split; masked when stored to LDS
  u32x4 kreg[K_IT], vreg[V_IT][2];
  auto row_off = [&](int key) -> int64_t {  // element offset of position key's row
    const int kk = min(key, kend - 1);
    return (((int64_t)phys_s[(kk - kbeg) / BS] * Hkv + g) * BS + kk % BS) * D;
  };
  auto gload = [&](int kt) {
    const int kv0 = kbeg + kt * BKV;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int e = tid + i * NT, key = e / (D / VE), c = e % (D / VE);
      kreg[i] = ld16(kc + row_off(kv0 + key) + c * VE);
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int e = tid + i * NT, kp = e % (BKV / 2), c = e / (BKV / 2);
      vreg[i][0] = ld16(vc + row_off(kv0 + 2 * kp) + c * VE);
      vreg[i][1] = ld16(vc + row_off(kv0 + 2 * kp + 1) + c * VE);
    }
  };
  const u32x4 zero = {0, 0, 0, 0};
  auto sstore = [&](int buf, int kt) {
    const int kv0 = kbeg + kt * BKV;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int e = tid + i * NT, key = e / (D / VE), c = e % (D / VE);
      st16(&Ks[buf][key * KLS + c * VE], kv0 + key < kend ? kreg[i] : zero);
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int e = tid + i * NT, kp = e % (BKV / 2), c = e / (BKV / 2);
      const u32x4 a = kv0 + 2 * kp < kend ? vreg[i][0] : zero;
      const u32x4 bb = kv0 + 2 * kp + 1 < kend ? vreg[i][1] : zero;
      T ea[VE], eb[VE];
      __builtin_memcpy(ea, &a, 16);
      __builtin_memcpy(eb, &bb, 16);
#pragma unroll
      for (int x = 0; x < VE; ++x) {
        typedef T pair_t __attribute__((ext_vector_type(2)));
        *reinterpret_cast<pair_t*>(&Vt[buf][(c * VE + x) * VLS + 2 * kp]) = pair_t{ea[x], eb[x]};
      }
    }
  };

  gload(0);
  sstore(0, 0);
  if (nt > 1) gload(1);
  __syncthreads();
  for (int kt = 0; kt < nt; ++kt) {
    const int cur = kt & 1;
    const int kv0 = kbeg + kt * BKV;
    if (wave_live && kv0 <= wave_lim) {
      // S^T = K Q^T (rows: keys, columns: this wave's query rows)
      f32x4 s[KTS][QS];
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[ks][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        Frag<T> kf[KTS];
#pragma unroll
        for (int ks = 0; ks < KTS; ++ks)
          kf[ks].load(&Ks[cur][(ks * 16 + fr) * KLS + dc * 32 + 8 * fg]);
#pragma unroll
        for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) s[ks][qs] = mfma_k32(kf[ks], qf[qs][dc], s[ks][qs]);
      }
      // mask (causal per row, split end), online softmax per query column
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const int lim = valid[qs] ? sq.first + tok[qs] : -1;  // last visible position
        float mx = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kv0 + ks * 16 + 4 * fg + j;
            const float val = (key <= lim && key < kend) ? s[ks][qs][j] * scale_log2 : -INFINITY;
            s[ks][qs][j] = val;
            mx = fmaxf(mx, val);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_i[qs], mx);
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_i[qs] - m_new);
        float ls = 0.f;
#pragma unroll
        for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = s[ks][qs][j] == -INFINITY ? 0.f : exp2f(s[ks][qs][j] - m_new);
            s[ks][qs][j] = p;
            ls += p;
          }
        l_i[qs] = l_i[qs] * alpha + ls;
        m_i[qs] = m_new;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) o[ds][qs] *= alpha;
      }
      // O^T += V^T P^T (the key order inside a k-group matches on both sides)
#pragma unroll
      for (int kc2 = 0; kc2 < KC; ++kc2) {
        Frag<T> pf[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) scores_to_frag(pf[qs], s[2 * kc2][qs], s[2 * kc2 + 1][qs]);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          Frag<T> vf;
          const T* row = &Vt[cur][(ds * 16 + fr) * VLS + kc2 * 32 + 4 * fg];
          load_split_frag(vf, row, row + 16);
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) o[ds][qs] = mfma_k32(vf, pf[qs], o[ds][qs]);
        }
      }
    }
    if (kt + 1 < nt) sstore(cur ^ 1, kt + 1);
    __syncthreads();
    if (kt + 2 < nt) gload(kt + 2);
  }

  // ---- partials of every valid row: o (unnormalised), m (log2 units), l
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    float l = l_i[qs];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (!valid[qs]) continue;
    const int64_t row = (int64_t)(sq.q0 + tok[qs]) * Hq + head[qs];
    if (row_splits(sq.first + tok[qs], ck, max_sp) == 1) {
      // the row's only split: its output, normalised (the combine skips it)
      if (sp == 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          store4(out + row * D + ds * 16 + 4 * fg, o[ds][qs][0] * inv, o[ds][qs][1] * inv,
                 o[ds][qs][2] * inv, o[ds][qs][3] * inv);
      }
      continue;
    }
    float* dst = ws + (row * max_sp + sp) * (D + 2);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      store4(dst + ds * 16 + 4 * fg, o[ds][qs][0], o[ds][qs][1], o[ds][qs][2], o[ds][qs][3]);
    if (fg == 0) {
      dst[D] = m_i[qs];
      dst[D + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow variant: at most 32 query rows per kv head (verification batches:
// q_len * G <= 32), where the wide kernel above is memory-latency bound (one
// tile in flight behind a workgroup barrier).  Here every wave runs its own
// key stream over the split -- 32-key steps w, w + 4, w + 8, ... -- for all
// 32 rows: K rows are loaded straight into the MFMA operand registers, V rows
// go through a wave-private LDS area to be transposed (pairs of keys written
// as 4-byte words), NB steps of loads are in flight per wave, and nothing in
// the key loop waits on another wave.  The four waves' (m, l, o) are merged
// through LDS at the end, and the split's partials go to the same workspace
// layout as the wide kernel's, for the same combine.
// ---------------------------------------------------------------------------

// DEPTH: wave steps in flight (2 measured best on the 7B verification batch:
// 5.6 TB/s against 5.5 and 5.4 for 3 and 4, with 4096-key splits, and 4.4 for
// one step in flight)
template <typename T, int D, int DEPTH = 2>
__global__ void __launch_bounds__(256, 1)
attn_paged_narrow_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                         const T* __restrict__ vc, const int32_t* __restrict__ bt, int max_blocks,
                         const int32_t* __restrict__ cu_q, const int32_t* __restrict__ ctx_lens,
                         int B, int Tq, int Hq, int Hkv, int BS, float scale_log2, int ck,
                         int max_qt,
                         int max_sp, int max_ctx, float* __restrict__ ws, int num_blocks,
                         T* __restrict__ out) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int QS = 2, KTS = kPnKeys / 16, DC = D / 32, DS = D / 16;
  constexpr int VLS = kPnKeys + VE;                      // padded V^T row (keys)
  constexpr int V_IT = (kPnKeys / 2) * (D / VE) / 64;    // key-pair loads per lane per step
  static_assert(V_IT * 64 == (kPnKeys / 2) * (D / VE), "V split");
  __shared__ __attribute__((aligned(16))) T Vt[4][D * VLS];
  __shared__ __attribute__((aligned(16))) float red_o[4][32][D + 4];
  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ int phys_s[kPnMaxSplitBlocks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int G = Hq / Hkv, QB = 32 / G;
  const int g = blockIdx.x % Hkv, item = blockIdx.x / Hkv;

  // ---- item -> (sequence, query tile, split), as in the wide kernel
  auto counts = [&](int bb, int& nqt, int& nsp) {
    const PgSeq s(cu_q, ctx_lens, bb, Tq, max_blocks, BS, max_ctx);
    nqt = s.ql > 0 ? min((s.ql + QB - 1) / QB, max_qt) : 0;
    nsp = s.ctx > 0 ? min((s.ctx + ck - 1) / ck, max_sp) : 0;
  };
  int b = -1, local = 0;
  for (int b0 = 0, base = 0; b0 < B; b0 += kWave) {
    int nqt = 0, nsp = 0;
    if (b0 + lane < B) counts(b0 + lane, nqt, nsp);
    const int n = nqt * nsp;
    int inc = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += y;
    }
    const int total = __shfl(inc, kWave - 1, kWave);
    if (item < base + total) {
      const bool mine = item >= base + inc - n && item < base + inc;
      const int L = __ffsll((unsigned long long)__ballot(mine)) - 1;
      b = b0 + L;
      local = item - base - __shfl(inc - n, L, kWave);
      break;
    }
    base += total;
  }
  if (b < 0) return;
  const PgSeq sq(cu_q, ctx_lens, b, Tq, max_blocks, BS, max_ctx);
  int nqt, nsp;
  counts(b, nqt, nsp);
  const int qt = local / nsp, sp = local % nsp;
  const int i_end = min(sq.ql, (qt + 1) * QB);
  const int kbeg = sp * ck;
  const int kend = min(min(sq.ctx, kbeg + ck), sq.first + i_end);
  if (kend <= kbeg) return;
  const int nb = (kend - kbeg + BS - 1) / BS;
  for (int i = tid; i < nb; i += 256) {  // up to kPnMaxSplitBlocks (512) entries
    const int p = bt[(int64_t)b * max_blocks + kbeg / BS + i];
    phys_s[i] = (p < 0 || p >= num_blocks) ? 0 : p;
  }

  // ---- the 32 query rows r = 16 qs + fr: token r / G of the tile, head r % G
  int tok[QS], lim[QS];
  bool valid[QS];
  Frag<T> qf[QS][DC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int r = 16 * qs + fr;
    tok[qs] = qt * QB + r / G;
    valid[qs] = tok[qs] < sq.ql;
    lim[qs] = valid[qs] ? sq.first + tok[qs] : -1;   // last visible position
    const int head = g * G + r % G;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (valid[qs])
        qf[qs][dc].load(q + ((int64_t)(sq.q0 + tok[qs]) * Hq + head) * D + dc * 32 + 8 * fg);
      else
        qf[qs][dc].zero();
    }
  }
  f32x4 o[DS][QS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) o[ds][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_i[QS], l_i[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    m_i[qs] = -INFINITY;
    l_i[qs] = 0.f;
  }
  __syncthreads();  // phys_s

  // ---- this wave's key steps: 32 keys starting at kbeg + 32 (4 j + wave)
  const int nsteps = (kend - kbeg + kPnKeys - 1) / kPnKeys;
  const int my_steps = nsteps > wave ? (nsteps - wave + 3) / 4 : 0;
  auto row_off = [&](int key) -> int64_t {  // element offset of position key's row (clamped)
    const int kk = min(key, kend - 1);
    return (((int64_t)phys_s[(kk - kbeg) / BS] * Hkv + g) * BS + kk % BS) * D;
  };
  struct Buf {
    Frag<T> k[KTS][DC];
    u32x4 v[V_IT][2];
  };
  auto gload = [&](Buf& bf, int j) {  // j: this wave's step index (past the end: reloads, unused)
    const int k0 = kbeg + kPnKeys * (4 * min(j, max(my_steps - 1, 0)) + wave);
#pragma unroll
    for (int ks = 0; ks < KTS; ++ks) {
      const int64_t ro = row_off(k0 + ks * 16 + fr);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) bf.k[ks][dc].load(kc + ro + dc * 32 + 8 * fg);
    }
#pragma unroll
    for (int u = 0; u < V_IT; ++u) {
      const int e = lane + 64 * u, kp = e % (kPnKeys / 2), c = e / (kPnKeys / 2);
      bf.v[u][0] = ld16(vc + row_off(k0 + 2 * kp) + c * VE);
      bf.v[u][1] = ld16(vc + row_off(k0 + 2 * kp + 1) + c * VE);
    }
  };
  T* vt = Vt[wave];
  const u32x4 zero = {0, 0, 0, 0};
  auto process = [&](const Buf& bf, int j) {
    const int k0 = kbeg + kPnKeys * (4 * j + wave);
    // S^T = K Q^T: rows keys k0 + 16 ks + 4 fg + jj, columns this lane's rows
    f32x4 sc[KTS][QS];
#pragma unroll
    for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        sc[ks][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) sc[ks][qs] = mfma_k32(bf.k[ks][dc], qf[qs][dc], sc[ks][qs]);
      }
    // V^T into this wave's LDS area (keys past the split stored as zeros)
#pragma unroll
    for (int u = 0; u < V_IT; ++u) {
      const int e = lane + 64 * u, kp = e % (kPnKeys / 2), c = e / (kPnKeys / 2);
      const u32x4 a = k0 + 2 * kp < kend ? bf.v[u][0] : zero;
      const u32x4 bb = k0 + 2 * kp + 1 < kend ? bf.v[u][1] : zero;
      T ea[VE], eb[VE];
      __builtin_memcpy(ea, &a, 16);
      __builtin_memcpy(eb, &bb, 16);
      typedef T pair_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int x = 0; x < VE; ++x)
        *reinterpret_cast<pair_t*>(&vt[(c * VE + x) * VLS + 2 * kp]) = pair_t{ea[x], eb[x]};
    }
    // online softmax per row (log2 domain)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = k0 + ks * 16 + 4 * fg + jj;
          const float val =
              (key <= lim[qs] && key < kend) ? sc[ks][qs][jj] * scale_log2 : -INFINITY;
          sc[ks][qs][jj] = val;
          mx = fmaxf(mx, val);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_i[qs], mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_i[qs] - m_new);
      float ls = 0.f;
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float pv = sc[ks][qs][jj] == -INFINITY ? 0.f : exp2f(sc[ks][qs][jj] - m_new);
          sc[ks][qs][jj] = pv;
          ls += pv;
        }
      l_i[qs] = l_i[qs] * alpha + ls;
      m_i[qs] = m_new;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) o[ds][qs] *= alpha;
    }
    // the V^T writes of every lane of this wave before the fragment reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T
    Frag<T> pf[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) scores_to_frag(pf[qs], sc[0][qs], sc[1][qs]);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      Frag<T> vf;
      const T* row = &vt[(ds * 16 + fr) * VLS + 4 * fg];
      load_split_frag(vf, row, row + 16);
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) o[ds][qs] = mfma_k32(vf, pf[qs], o[ds][qs]);
    }
    // every lane's fragment reads before the next step overwrites the area
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (my_steps > 0) {
    // whole groups of DEPTH steps: every iteration uses the buffers in the
    // order it refills them, so the loads in flight at the loop head are the
    // same on entry and on the back edge and no wait has to drain them; the
    // last group's refills (clamped past the end) are never used
    Buf bufs[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) gload(bufs[d], d);
    int j = 0;
    for (; j + DEPTH <= my_steps; j += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        process(bufs[d], j + d);
        gload(bufs[d], j + d + DEPTH);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (j + d < my_steps) process(bufs[d], j + d);
  }

  // ---- merge the four waves (fixed order) and write the split's partials
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    float l = l_i[qs];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int r = 16 * qs + fr;
    if (fg == 0) {
      red_m[wave][r] = m_i[qs];
      red_l[wave][r] = l;
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      *reinterpret_cast<f32x4*>(&red_o[wave][r][ds * 16 + 4 * fg]) = o[ds][qs];
  }
  __syncthreads();
  for (int idx = tid; idx < 32 * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    const int tk = qt * QB + r / G;
    if (tk >= sq.ql) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][r]);
    float oa = 0.f, la = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sw = red_m[w][r] == -INFINITY ? 0.f : exp2f(red_m[w][r] - M);
      oa += sw * red_o[w][r][d];
      la += sw * red_l[w][r];
    }
    const int64_t row = (int64_t)(sq.q0 + tk) * Hq + g * G + r % G;
    if (row_splits(sq.first + tk, ck, max_sp) == 1) {
      // the row's only split: its output, normalised (the combine skips it)
      if (sp == 0) out[row * D + d] = from_f32<T>(la > 0.f ? oa / la : 0.f);
      continue;
    }
    float* dst = ws + (row * max_sp + sp) * (D + 2);
    dst[d] = oa;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = la;
    }
  }
}

// Merge the splits of one (query token, head) in fixed order.  Token t's
// sequence is found by binary search over cu_q; its row saw splits
// 0 .. ceil((p_t + 1) / ck) - 1.  A row with one split was written by the
// attention kernel itself.
template <typename T, int D>
__global__ void __launch_bounds__(kCombineThreads)
attn_paged_combine(const float* __restrict__ ws, const int32_t* __restrict__ cu_q,
                   const int32_t* __restrict__ ctx_lens, int B, int Tq, int Hq, int BS,
                   int max_blocks, int ck, int max_sp, int max_ctx, T* __restrict__ out) {
  const int h = blockIdx.x, t = blockIdx.y;
  int lo = cu_q ? 0 : t, hi = B;  // largest b with cu_q[b] <= t
  while (cu_q && hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= t) lo = mid;
    else hi = mid;
  }
  const PgSeq sq(cu_q, ctx_lens, lo, Tq, max_blocks, BS, max_ctx);
  const int ns = row_splits(sq.first + (t - sq.q0), ck, max_sp);
  if (ns == 1) return;  // written by the attention kernel
  combine_row<T, D>(ws + ((int64_t)t * Hq + h) * max_sp * (D + 2), ns,
                    out + ((int64_t)t * Hq + h) * D);
}

template <typename T, int D>
static hipError_t launch_paged(const T* q, const T* kc, const T* vc, const int32_t* bt,
                               int max_blocks, const int32_t* cu_q, const int32_t* ctx, int B,
                               int Tq, int Hq, int Hkv, int BS, float sl2, int max_ctx,
                               const PagedPlan& pl, float* ws, T* out, int num_blocks,
                               hipStream_t st) {
  const long wgs = (long)B * pl.max_qt * pl.max_sp * Hkv;
  if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
  if (pl.narrow)
    hipLaunchKernelGGL((attn_paged_narrow_kernel<T, D>), dim3((unsigned)wgs), dim3(256), 0, st, q,
                       kc, vc, bt, max_blocks, cu_q, ctx, B, Tq, Hq, Hkv, BS, sl2, pl.ck, pl.max_qt,
                       pl.max_sp, max_ctx, ws, num_blocks, out);
  else
    hipLaunchKernelGGL((attn_paged_kernel<T, D>), dim3((unsigned)wgs), dim3(256), 0, st, q, kc,
                       vc, bt, max_blocks, cu_q, ctx, B, Tq, Hq, Hkv, BS, sl2, pl.ck, pl.max_qt,
                       pl.max_sp, max_ctx, ws, num_blocks, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_paged_combine<T, D>), dim3(Hq, Tq), dim3(kCombineThreads), 0, st, ws, cu_q, ctx, B,
                     Tq, Hq, BS, max_blocks, pl.ck, pl.max_sp, max_ctx, out);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_paged_qlens(const T* q, const T* k_cache, const T* v_cache,
                            const int32_t* block_table, int max_blocks, const int32_t* cu_q,
                            const int32_t* context_lens, int B, int Tq, int Hq, int Hkv, int D,
                            int BS, int max_context_len, float scale, T* out, const PagedPlan& pl,
                            void* ws, int num_blocks, hipStream_t st) {
  if (B == 0 || Tq == 0 || pl.max_qt == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  float* w = reinterpret_cast<float*>(ws);
  if (D == 128)
    return launch_paged<T, 128>(q, k_cache, v_cache, block_table, max_blocks, cu_q, context_lens,
                                B, Tq, Hq, Hkv, BS, sl2, max_context_len, pl, w, out, num_blocks,
                                st);
  if (D == 64)
    return launch_paged<T, 64>(q, k_cache, v_cache, block_table, max_blocks, cu_q, context_lens,
                               B, Tq, Hq, Hkv, BS, sl2, max_context_len, pl, w, out, num_blocks,
                               st);
  return hipErrorInvalidValue;
}

// The decode step (one new token per sequence) through the narrow kernel.
template <typename T>
hipError_t attn_decode_narrow(const T* q, const T* k_cache, const T* v_cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                              int max_context_len, float scale, T* out, int ck, int max_sp,
                              void* ws, int num_blocks, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  float* w = reinterpret_cast<float*>(ws);
  const long wgs = (long)B * max_sp * Hkv;
  if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
  if (D == 128) {
    hipLaunchKernelGGL((attn_paged_narrow_kernel<T, 128>), dim3((unsigned)wgs), dim3(256), 0, st,
                       q, k_cache, v_cache, block_table, max_blocks, nullptr, context_lens, B, B,
                       Hq, Hkv, BS, sl2, ck, 1, max_sp, max_context_len, w, num_blocks, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_paged_combine<T, 128>), dim3(Hq, B), dim3(kCombineThreads), 0, st, w, nullptr,
                       context_lens, B, B, Hq, BS, max_blocks, ck, max_sp, max_context_len, out);
  } else if (D == 64) {
    hipLaunchKernelGGL((attn_paged_narrow_kernel<T, 64>), dim3((unsigned)wgs), dim3(256), 0, st,
                       q, k_cache, v_cache, block_table, max_blocks, nullptr, context_lens, B, B,
                       Hq, Hkv, BS, sl2, ck, 1, max_sp, max_context_len, w, num_blocks, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_paged_combine<T, 64>), dim3(Hq, B), dim3(kCombineThreads), 0, st, w, nullptr,
                       context_lens, B, B, Hq, BS, max_blocks, ck, max_sp, max_context_len, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t attn_decode_narrow<bf16>(const bf16*, const bf16*, const bf16*,
                                             const int32_t*, int, const int32_t*, int, int, int,
                                             int, int, int, float, bf16*, int, int, void*, int,
                                             hipStream_t);
template hipError_t attn_decode_narrow<float>(const float*, const float*, const float*,
                                              const int32_t*, int, const int32_t*, int, int, int,
                                              int, int, int, float, float*, int, int, void*, int,
                                              hipStream_t);

template hipError_t attn_paged_qlens<bf16>(const bf16*, const bf16*, const bf16*, const int32_t*,
                                           int, const int32_t*, const int32_t*, int, int, int,
                                           int, int, int, int, float, bf16*, const PagedPlan&,
                                           void*, int, hipStream_t);
template hipError_t attn_paged_qlens<float>(const float*, const float*, const float*,
                                            const int32_t*, int, const int32_t*, const int32_t*,
                                            int, int, int, int, int, int, int, float, float*,
                                            const PagedPlan&, void*, int, hipStream_t);

}  // namespace dl
