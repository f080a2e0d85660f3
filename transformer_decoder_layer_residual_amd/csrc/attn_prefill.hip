// attn_prefill.hip -- causal, variable-length, grouped-query flash attention
// for prefill (gfx950 MFMA).
//
// What it computes: for every packed sequence b (rows cu_seqlens[b] ..
// cu_seqlens[b+1]-1), every query head h and every query row i, the softmax of
// scale * q_i . k_j over the keys j <= i of the same sequence, applied to V.
// K/V head = h / (Hq / Hkv).  Prefill sends the whole sequence through a
// single attention kernel that never writes the score matrix to memory (ATB
// fusion-strategy page, "Attention fusion"; ops-transformer Llama2-7B page,
// "KV cache and operators": prefill runs the full sequence through
// FlashAttention).
//
// Layout: q [T][Hq][D], k/v [T][Hkv][D], out [T][Hq][D].
//
// Mapping: one workgroup = 4 waves x QW query rows of one head; keys are
// streamed in tiles of 64 through LDS (K row-major, V transposed so the PV
// operand reads are contiguous).  The MFMA computes S^T = K Q^T so each lane
// owns one query column: the row statistics of the online softmax reduce in
// registers plus two cross-lane steps, P^T feeds the PV MFMA straight from
// the score registers (the key order inside an MFMA k-group is permuted the
// same way for both operands), and O^T accumulates with one query per lane,
// which makes the rescale by exp2(m_old - m_new) a per-lane multiply.
#include "dl_internal.hpp"

namespace dl {

__device__ __forceinline__ void make_frag(Frag<bf16>& f, f32x4 a, f32x4 b) {
  f.v = bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
               (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}
__device__ __forceinline__ void make_frag(Frag<float>& f, f32x4 a, f32x4 b) {
  f.lo = a;
  f.hi = b;
}
__device__ __forceinline__ void load_frag2(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p0);
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(p1);
  f.v = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
__device__ __forceinline__ void load_frag2(Frag<float>& f, const float* p0, const float* p1) {
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
}

template <typename T>
struct Pair2 {
  typedef T type __attribute__((ext_vector_type(2)));
};

constexpr int kPfWaves = 4;
constexpr int kPfBKV = 64;

template <typename T, int D, int QW>
__global__ void __launch_bounds__(kPfWaves * kWave)
attn_prefill_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2,
                    T* __restrict__ out, int n_qtiles) {
  constexpr int NT = kPfWaves * kWave, BQ = kPfWaves * QW, BKV = kPfBKV;
  constexpr int QS = QW / 16, KTS = BKV / 16, DC = D / 32, DS = D / 16, KC = BKV / 32;
  constexpr int VE = 16 / sizeof(T);
  constexpr int KLS = D + VE;        // padded K row (16 B)
  constexpr int VLS = BKV + VE;      // padded V^T row (16 B)
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KLS];
  __shared__ __attribute__((aligned(16))) T Vt[D * VLS];

  const int b = blockIdx.z, h = blockIdx.y;
  const int qt = n_qtiles - 1 - (int)blockIdx.x;  // heavy (late) tiles first
  const int t0 = cu[b], S = cu[b + 1] - t0;
  const int q_begin = qt * BQ;
  if (q_begin >= S) return;
  const int g = h / (Hq / Hkv);
  const int kv_end = min(S, q_begin + BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int qw0 = q_begin + wave * QW;

  Frag<T> qf[QS][DC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qi = qw0 + qs * 16 + fr;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (qi < S)
        qf[qs][dc].load(q + ((int64_t)(t0 + qi) * Hq + h) * D + dc * 32 + 8 * fg);
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

  const u32x4 zero = {0, 0, 0, 0};
  for (int kt = 0; kt < nkv; ++kt) {
    const int kv0 = kt * BKV;
    __syncthreads();
    // K tile, row-major
    for (int i = tid; i < BKV * (D / VE); i += NT) {
      const int key = i / (D / VE), c = i % (D / VE);
      const u32x4 val = (kv0 + key < kv_end)
                            ? ld16(k + ((int64_t)(t0 + kv0 + key) * Hkv + g) * D + c * VE)
                            : zero;
      st16(Ks + key * KLS + c * VE, val);
    }
    // V tile, transposed: each thread takes two adjacent keys and VE d-values
    for (int i = tid; i < (BKV / 2) * (D / VE); i += NT) {
      const int kp = i % (BKV / 2), c = i / (BKV / 2);
      const int key0 = 2 * kp;
      const u32x4 a = (kv0 + key0 < kv_end)
                          ? ld16(v + ((int64_t)(t0 + kv0 + key0) * Hkv + g) * D + c * VE)
                          : zero;
      const u32x4 bb = (kv0 + key0 + 1 < kv_end)
                           ? ld16(v + ((int64_t)(t0 + kv0 + key0 + 1) * Hkv + g) * D + c * VE)
                           : zero;
      T ea[VE], eb[VE];
      __builtin_memcpy(ea, &a, 16);
      __builtin_memcpy(eb, &bb, 16);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        typename Pair2<T>::type pr = {ea[e], eb[e]};
        *reinterpret_cast<typename Pair2<T>::type*>(Vt + (c * VE + e) * VLS + key0) = pr;
      }
    }
    __syncthreads();

    // S^T = K Q^T  (rows: keys, cols: queries)
    f32x4 s[KTS][QS];
#pragma unroll
    for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) s[ks][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      Frag<T> kf[KTS];
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks) kf[ks].load(Ks + (ks * 16 + fr) * KLS + dc * 32 + 8 * fg);
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[ks][qs] = mfma_k32(kf[ks], qf[qs][dc], s[ks][qs]);
    }

    // causal mask, scale (log2 domain), online softmax per query column
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int qi = qw0 + qs * 16 + fr;
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kv0 + ks * 16 + 4 * fg + j;
          const float val = (key <= qi && key < kv_end) ? s[ks][qs][j] * scale_log2 : -INFINITY;
          s[ks][qs][j] = val;
          mx = fmaxf(mx, val);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_i[qs], mx);
      const float alpha = exp2f(m_i[qs] - m_new);
      float ls = 0.f;
#pragma unroll
      for (int ks = 0; ks < KTS; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = exp2f(s[ks][qs][j] - m_new);
          s[ks][qs][j] = p;
          ls += p;
        }
      l_i[qs] = l_i[qs] * alpha + ls;
      m_i[qs] = m_new;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) o[ds][qs] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      Frag<T> pf[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) make_frag(pf[qs], s[2 * kc][qs], s[2 * kc + 1][qs]);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        Frag<T> vf;
        const T* row = Vt + (ds * 16 + fr) * VLS + kc * 32 + 4 * fg;
        load_frag2(vf, row, row + 16);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) o[ds][qs] = mfma_k32(vf, pf[qs], o[ds][qs]);
      }
    }
  }

#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    float l = l_i[qs];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = 1.0f / l;
    const int qi = qw0 + qs * 16 + fr;
    if (qi < S) {
      T* dst = out + ((int64_t)(t0 + qi) * Hq + h) * D + 4 * fg;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        store4(dst + ds * 16, o[ds][qs][0] * inv, o[ds][qs][1] * inv, o[ds][qs][2] * inv,
               o[ds][qs][3] * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel on v_mfma_f32_32x32x16_bf16.  4 waves x 32 queries; KV tiles of
// 64 keys double-buffered in LDS, the next tile's loads in registers while the
// current tile is processed (one barrier per tile).  S^T = K Q^T puts one
// query per lane column (rows of the 32x32 block are keys 8i + 4(l/32) + j),
// so the row statistics need one cross-lane step; P^T feeds the PV MFMA from
// the score registers with the key order of its k-slots matched by the V^T
// reads.  Waves skip tiles entirely above their causal diagonal.  Blocks are
// ordered so that every q-tile of a head runs on the same XCD (K/V of a head
// stay in that XCD's L2).  When the whole grid is resident at once (two
// workgroups per CU), the heavier half of the q-tiles goes first, heaviest
// first, then the lighter half lightest first: a CU then holds tiles t and
// n-1-t, whose causal work adds up to the same total on every CU
// (heaviest-first alone paired heavy with middle tiles: up to 1.4x the
// average work on one CU; 4% slower at 7B B1 x 2048).  A larger grid is
// dispatched as slots free up, and there heaviest-first throughout balances
// better (the 8B batch of 8 ragged sequences: 106 against 114 us).
// ---------------------------------------------------------------------------
// workgroups of the bf16 kernel resident at once: two per CU on 256 CUs
constexpr long kPfResidentBlocks = 2 * 256;

// Column of key `key` in a V^T tile row.  Within each 16-key group the
// 32x32x16 score block gives a lane keys {4h..4h+3} and {8+4h..8+4h+3} (h =
// lane / 32) of one k16 step; swapping bits 2 and 3 of the key puts those
// eight keys side by side, so the P.V operand is one 16-byte LDS read.
__device__ __forceinline__ int vt_col(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_prefill_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                         const bf16* __restrict__ v, const int32_t* __restrict__ cu, int Hq,
                         int Hkv, float scale_log2, bf16* __restrict__ out, int n_qtiles,
                         int n_heads_total, int pair_order) {
  constexpr int BQ = 128, BKV = 64, QW = 32;
  constexpr int KLS = D + 8;          // padded K row (elements)
  constexpr int VLS = BKV + 8;        // padded V^T row
  constexpr int DK = D / 16;          // k16 steps over D
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int K_IT = BKV * (D / 8) / 256;           // 16-byte K loads per thread
  constexpr int V_IT = (BKV / 2) * (D / 8) / 256;     // key-pair V loads per thread
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BKV * KLS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * VLS];

  // ---- block -> (q-tile, head): XCD-aware when the head count allows
  const int L = blockIdx.x;
  int u, hh;                                            // u: rank of the q-tile in launch order
  if ((n_heads_total & 7) == 0) {
    const int xcd = L & 7, idx = L >> 3;
    const int hpx = n_heads_total >> 3;                 // heads per XCD
    u = idx / hpx;
    hh = xcd * hpx + idx % hpx;
  } else {
    u = L / n_heads_total;
    hh = L % n_heads_total;
  }
  const int heavy = (n_qtiles + 1) / 2;
  const int qt = !pair_order || u < heavy ? n_qtiles - 1 - u : u - heavy;
  const int b = hh / Hq, h = hh % Hq;
  const int t0 = cu[b], S = cu[b + 1] - t0;
  const int q_begin = qt * BQ;
  if (q_begin >= S) return;
  const int g = h / (Hq / Hkv);
  const int kv_end = min(S, q_begin + BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int qw0 = q_begin + wave * QW;
  const int qi = qw0 + fr;                              // this lane's query

  bf16x8 qf[DK];
#pragma unroll
  for (int ds = 0; ds < DK; ++ds) {
    if (qi < S)
      qf[ds] = *reinterpret_cast<const bf16x8*>(q + ((int64_t)(t0 + qi) * Hq + h) * D + ds * 16 + 8 * fh);
    else
      qf[ds] = bf16x8{};
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_i = -INFINITY, l_i = 0.f;

  // ---- K/V tile loads (registers) and LDS stores
  u32x4 kreg[K_IT], vreg[V_IT][2];
  const u32x4 zero = {0, 0, 0, 0};
  auto gload = [&](int kt) {
    const int kv0 = kt * BKV;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int e = tid + i * 256, key = e / (D / 8), c = e % (D / 8);
      kreg[i] = (kv0 + key < kv_end)
                    ? ld16(k + ((int64_t)(t0 + kv0 + key) * Hkv + g) * D + c * 8) : zero;
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int e = tid + i * 256, kp = e % (BKV / 2), c = e / (BKV / 2);
      const int key0 = kv0 + 2 * kp;
      vreg[i][0] = (key0 < kv_end) ? ld16(v + ((int64_t)(t0 + key0) * Hkv + g) * D + c * 8) : zero;
      vreg[i][1] = (key0 + 1 < kv_end) ? ld16(v + ((int64_t)(t0 + key0 + 1) * Hkv + g) * D + c * 8) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int e = tid + i * 256, key = e / (D / 8), c = e % (D / 8);
      st16(&Ks[buf][key * KLS + c * 8], kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int e = tid + i * 256, kp = e % (BKV / 2), c = e / (BKV / 2);
      bf16 a[8], bb[8];
      __builtin_memcpy(a, &vreg[i][0], 16);
      __builtin_memcpy(bb, &vreg[i][1], 16);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2*>(&Vt[buf][(c * 8 + x) * VLS + vt_col(2 * kp)]) = bf16x2{a[x], bb[x]};
      }
    }
  };

  gload(0);
  sstore(0);
  if (nkv > 1) gload(1);
  __syncthreads();
  for (int kt = 0; kt < nkv; ++kt) {
    const int cur = kt & 1;
    const int kv0 = kt * BKV;
    if (kv0 <= qw0 + QW - 1) {           // otherwise every key of the tile is in this wave's future
      // S^T = K Q^T: two 32-key blocks as two independent MFMA chains,
      // interleaved, with the K fragments read two k16 steps ahead (a single
      // chain with each read just before its MFMA waited on both latencies)
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      auto kfrag = [&](int kb, int ds) {
        return *reinterpret_cast<const bf16x8*>(&Ks[cur][(kb * 32 + fr) * KLS + ds * 16 + 8 * fh]);
      };
      bf16x8 kf[3][2];
      kf[0][0] = kfrag(0, 0);
      kf[0][1] = kfrag(1, 0);
      kf[1][0] = kfrag(0, 1);
      kf[1][1] = kfrag(1, 1);
#pragma unroll
      for (int ds = 0; ds < DK; ++ds) {
        if (ds + 2 < DK) {
          kf[(ds + 2) % 3][0] = kfrag(0, ds + 2);
          kf[(ds + 2) % 3][1] = kfrag(1, ds + 2);
        }
        sc[0] = mfma_32x32x16(kf[ds % 3][0], qf[ds], sc[0]);
        sc[1] = mfma_32x32x16(kf[ds % 3][1], qf[ds], sc[1]);
      }
      // V^T fragments of the first P.V step, read while the softmax runs
      auto vfrag = [&](int step, int db) {
        const int kbase = (step >> 1) * 32 + 16 * (step & 1) + 8 * fh;
        return *reinterpret_cast<const bf16x8*>(&Vt[cur][(db * 32 + fr) * VLS + kbase]);
      };
      bf16x8 vf[2][DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[0][db] = vfrag(0, db);
      // mask + online softmax for this lane's query.  The running max m_i is
      // kept in the log2 domain (scaled); the raw scores' max is scaled once
      // (the scale is positive) and each weight is exp2(fma(s, scale, -m)).
      // A tile whose every key is visible to every query of the wave needs
      // no mask.  The softmax is the VALU-heavy part of the loop (a wave64
      // VALU op takes four cycles against an MFMA's 32 per 32x32x16 block),
      // so every op saved here is kept out of the MFMAs' way.
      float mx = -INFINITY;
      if (kv0 + BKV - 1 <= qw0 && kv0 + BKV <= kv_end) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kv0 + kb * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
            const float val = (key <= qi && key < kv_end) ? sc[kb][e] : -INFINITY;
            sc[kb][e] = val;
            mx = fmaxf(mx, val);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_i, mx * scale_log2);
      // v_exp_f32 directly: arguments are <= 0 here, and results below the
      // normal range (weights under 2^-126) may flush to zero
      const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e], scale_log2, -m_new));
          sc[kb][e] = p;
          ls += p;
        }
      l_i = l_i * alpha + ls;
      // rescale O only when some lane's running max moved (alpha == 1 leaves
      // O unchanged, and later tiles rarely raise the max)
      if (__ballot(m_new != m_i)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      m_i = m_new;
      // O^T += V^T P^T in four k16 steps (kb, s2); step i+1's V^T fragments
      // are read while step i's MFMAs run.  Keys kb*32 + 16*s2 + {4fh..4fh+3,
      // 8+4fh..8+4fh+3} are eight adjacent V^T columns after vt_col's
      // permutation, so each fragment is one 16-byte read.
#pragma unroll
      for (int step = 0; step < 4; ++step) {
        const int kb = step >> 1, s2 = step & 1;
        if (step + 1 < 4) {
#pragma unroll
          for (int db = 0; db < DB; ++db) vf[(step + 1) & 1][db] = vfrag(step + 1, db);
        }
        const bf16x8 pf = {(bf16)sc[kb][8 * s2], (bf16)sc[kb][8 * s2 + 1], (bf16)sc[kb][8 * s2 + 2],
                           (bf16)sc[kb][8 * s2 + 3], (bf16)sc[kb][8 * s2 + 4], (bf16)sc[kb][8 * s2 + 5],
                           (bf16)sc[kb][8 * s2 + 6], (bf16)sc[kb][8 * s2 + 7]};
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma_32x32x16(vf[step & 1][db], pf, o[db]);
      }
    }
    if (kt + 1 < nkv) sstore(cur ^ 1);
    __syncthreads();
    if (kt + 2 < nkv) gload(kt + 2);
  }

  float l = l_i + __shfl_xor(l_i, 32, kWave);
  const float inv = 1.0f / l;
  if (qi < S) {
    bf16* dst = out + ((int64_t)(t0 + qi) * Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store4(dst + db * 32 + 8 * i + 4 * fh, o[db][4 * i] * inv, o[db][4 * i + 1] * inv,
               o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
  }
}

template <typename T>
hipError_t attn_prefill(const T* q, const T* k, const T* v, const int32_t* cu_seqlens, int B,
                        int max_seqlen, int Hq, int Hkv, int D, float scale, T* out,
                        hipStream_t st) {
  constexpr int QW = 32;
  constexpr int BQ = kPfWaves * QW;
  if (B == 0 || max_seqlen == 0) return hipSuccess;
  const int n_qtiles = (max_seqlen + BQ - 1) / BQ;
  const float sl2 = scale * 1.4426950408889634f;
  if constexpr (sizeof(T) == 2) {
    const int nh = B * Hq;
    dim3 grid(n_qtiles * nh), block(256);
    const int pair = (long)n_qtiles * nh <= kPfResidentBlocks ? 1 : 0;
    if (D == 128)
      hipLaunchKernelGGL((attn_prefill_bf16_kernel<128>), grid, block, 0, st, q, k, v, cu_seqlens,
                         Hq, Hkv, sl2, out, n_qtiles, nh, pair);
    else if (D == 64)
      hipLaunchKernelGGL((attn_prefill_bf16_kernel<64>), grid, block, 0, st, q, k, v, cu_seqlens,
                         Hq, Hkv, sl2, out, n_qtiles, nh, pair);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  dim3 grid(n_qtiles, Hq, B), block(kPfWaves * kWave);
  if (D == 128)
    hipLaunchKernelGGL((attn_prefill_kernel<T, 128, QW>), grid, block, 0, st, q, k, v, cu_seqlens,
                       Hq, Hkv, sl2, out, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL((attn_prefill_kernel<T, 64, QW>), grid, block, 0, st, q, k, v, cu_seqlens,
                       Hq, Hkv, sl2, out, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template hipError_t attn_prefill<bf16>(const bf16*, const bf16*, const bf16*, const int32_t*, int,
                                       int, int, int, int, float, bf16*, hipStream_t);
template hipError_t attn_prefill<float>(const float*, const float*, const float*, const int32_t*,
                                        int, int, int, int, int, float, float*, hipStream_t);

}  // namespace dl
