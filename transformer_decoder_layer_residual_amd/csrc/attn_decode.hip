// attn_decode.hip -- paged grouped-query decode attention (gfx950).
//
// What it computes: one new query row per sequence b (q [B][Hq][D]); for each
// query head h the softmax of scale * q . k_j over the cached positions
// j = 0 .. context_lens[b]-1, applied to V.  Position j lives in physical
// block block_table[b][j / BS], slot j % BS, of a [num_blocks][Hkv][BS][D]
// cache (ATB KV-cache page, "KV cache memory bottleneck": paged blocks,
// block_table, contextLens; ops-transformer Llama2-7B page, "KV cache and
// operators": at decode Q is [1, heads, 1, dim] and K/V come from the cache,
// with a decode-specialised kernel instead of the tiled one).
//
// Design (HBM-bound: every cached K/V byte is read exactly once):
//   * one workgroup per (sequence, kv head, split); a split is a fixed range
//     of LOGICAL blocks, so the arithmetic does not depend on which physical
//     blocks hold the data (a permuted block_table gives bit-identical
//     results); the splits of all sequences are numbered densely, so with
//     ragged contexts no idle workgroups sit between working ones (measured:
//     idle ones in between cost about a fifth of the bandwidth);
//   * the whole query group (Hq/Hkv heads sharing the kv head) is handled by
//     the workgroup, so each K/V byte serves all of them;
//   * each KV block is read straight into registers with 16-byte loads (a
//     block of one head is one contiguous BS x D run); for query groups of
//     up to two heads two blocks are in flight, and the physical ids of the
//     split's blocks are fetched once, up front, so no load waits on a
//     block-table read;
//   * scores: each thread holds a 16-byte slice of a token row; partial dots
//     of all group heads are reduced over the token's lanes with shuffles;
//   * online softmax in the log2 domain, kept per wave over the tokens the
//     wave owns, so the block loop needs no barrier; waves merge once;
//   * each split writes (o, m, l) in fp32; a second kernel combines the
//     splits in fixed order.
//
// INT8 cache (ATB KV-cache page, section "KV cache quantisation": the paged
// attention dequantises the blocks as it loads them; one fp32 scale per
// token row of K and of V): each thread reads a slice of codes (16 bytes,
// or 8 for query groups of more than two heads) and the row's scale.  A code byte c is read as the unsigned byte u = c + 128
// (one XOR per four codes, then one byte-to-float convert per code), so
//   q . k = s_k * (sum_d q_d u_d - 128 * sum_d q_d)
//   sum_j p_j v_j = sum_j (p_j s_v,j) u_j - 128 * sum_j p_j s_v,j
// where the query sums are taken once per thread and the second correction
// is carried next to the softmax denominator.
#include <type_traits>

#include "attn_combine.hpp"
#include "dl_internal.hpp"

namespace dl {

constexpr int kDecThreads = 256;
constexpr int kDecMaxBS = 128;
constexpr int kDecMaxSplitBlocks = 8;  // KV blocks per split, at most

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int max_context_len, int BS) {
  DecodePlan pl{};
  const int nblk = (max_context_len + BS - 1) / BS;
  const int items = B * Hkv;
  // aim for >= 2048 workgroups at the longest context, at most 8 blocks each
  int want = (2048 + items - 1) / items;
  int cb = (nblk + want - 1) / want;
  if (cb > kDecMaxSplitBlocks) cb = kDecMaxSplitBlocks;
  if (cb < 2 && nblk >= 16) cb = 2;
  if (cb < 1) cb = 1;
  pl.chunk_blocks = cb;
  pl.max_splits = nblk > 0 ? (nblk + cb - 1) / cb : 1;
  pl.ws_bytes = (size_t)B * Hq * pl.max_splits * (D + 2) * sizeof(float);
  // Query groups of 4 or 8 heads with enough work go through the narrow
  // paged kernel (MFMA over the group's rows): every thread of this kernel
  // would hold G x D of state and reduce G partial dots per token with lane
  // shuffles, which held it to 1.5 TB/s at 70B (G 8) and 3.6-4.0 TB/s at 8B
  // B64 (G 4) against 4.6 and 4.3 TB/s for the narrow kernel.  Below 131072
  // (kv head, key) pairs at the longest context this kernel stays faster
  // (8B B8 at contexts up to 1100: 11 us against 13 us).
  const int G = Hq / Hkv;
  if (G >= 4 && (double)B * Hkv * max_context_len >= 131072.0) {
    pl.narrow_ck = narrow_split(B, Hkv, max_context_len, BS);
    pl.narrow_sp = (max_context_len + pl.narrow_ck - 1) / pl.narrow_ck;
    const size_t w = (size_t)B * Hq * pl.narrow_sp * (D + 2) * sizeof(float);
    if (w > pl.ws_bytes) pl.ws_bytes = w;
  }
  return pl;
}

// How a thread reads its SB-byte slice of a cached row.
template <typename T, typename KV, int SB>
struct DecSlice {  // cache in the layer dtype: 16-byte slices
  static_assert(SB == 16, "layer-dtype caches are read in 16-byte slices");
  static constexpr bool kQ8 = false;
  static constexpr int VE = 16 / sizeof(T);
  using L = u32x4;
  static __device__ __forceinline__ L load(const KV* p) { return ld16(p); }
  static __device__ __forceinline__ void unpack(L v, float* f) { unpack16(v, f, T()); }
};
template <typename T, int SB>
struct DecSlice<T, int8_t, SB> {  // INT8 codes, read as code + 128
  static_assert(SB == 8 || SB == 16, "INT8 slices are 8 or 16 bytes");
  static constexpr bool kQ8 = true;
  static constexpr int VE = SB;
  using L = typename std::conditional<SB == 16, u32x4, u32x2>::type;
  static __device__ __forceinline__ L load(const int8_t* p) {
    if constexpr (SB == 16) return ld16(p);
    else return ld8(p);
  }
  static __device__ __forceinline__ void unpack(L v, float* f) {
#pragma unroll
    for (int i = 0; i < SB / 4; ++i) {
      const uint32_t w = v[i] ^ 0x80808080u;
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * i + e] = (float)((w >> (8 * e)) & 0xffu);
    }
  }
};

// SB: bytes of a row slice per thread; DEPTH: KV blocks in flight (query
// groups of up to two heads).
template <typename T, typename KV, int D, int G, int SB, int DEPTH>
__global__ void __launch_bounds__(kDecThreads)
attn_decode_kernel(const T* __restrict__ q, const KV* __restrict__ kc, const KV* __restrict__ vc,
                   const float* __restrict__ ksc, const float* __restrict__ vsc,
                   const int32_t* __restrict__ bt, int max_blocks, const int32_t* __restrict__ ctx,
                   int B, int Hq, int Hkv, int BS, float scale_log2, int chunk_blocks,
                   int max_splits, float* __restrict__ ws, int num_blocks) {
  // Register-resident streaming: thread t owns 16-byte chunk c = t % LPT of
  // tokens tok = t / LPT + TPI * i (i = 0 .. NI-1) of every KV block, for K
  // and V alike.  Scores are reduced over the LPT lanes of a token with lane
  // shuffles; every wave keeps its own online softmax (m, l, o) over the
  // tokens it owns, so the block loop has no workgroup barrier; the four
  // waves are merged once at the end of the split.
  using Sl = DecSlice<T, KV, SB>;
  using Ld = typename Sl::L;
  constexpr bool Q8 = Sl::kQ8;
  constexpr int NT = kDecThreads, VE = Sl::VE;
  constexpr int QE = 16 / sizeof(T);           // query elements per 16-byte load
  constexpr int LPT = D / VE;                 // lanes per token row
  constexpr int TPI = NT / LPT;               // tokens per load step (whole workgroup)
  constexpr int NI = (kDecMaxBS + TPI - 1) / TPI;
  constexpr int NWV = NT / kWave;
  __shared__ float red_m[NWV][G], red_l[NWV][G];
  __shared__ __attribute__((aligned(16))) float red_o[NWV][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // lengths beyond the table or the host-declared maximum are clamped, so a
  // violated precondition cannot index outside block_table or the workspace
  auto blocks_of = [&](int len) {
    return min(min((len + BS - 1) / BS, max_blocks), max_splits * chunk_blocks);
  };
  // Workgroup -> (kv head, work item); work items are the sequences' splits
  // numbered in order, found by a wave prefix sum over the split counts.
  // The grid is sized for the longest context, so the unused workgroups all
  // sit at its end instead of leaving holes between working ones.
  const int g = blockIdx.x % Hkv, item = blockIdx.x / Hkv;
  int b = -1, split = 0;
  for (int b0 = 0, base = 0; b0 < B; b0 += kWave) {
    const int nb_l = b0 + lane < B ? blocks_of(ctx[b0 + lane]) : 0;
    const int ns = (nb_l + chunk_blocks - 1) / chunk_blocks;
    int inc = ns;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += y;
    }
    const int total = __shfl(inc, kWave - 1, kWave);
    if (item < base + total) {
      const bool mine = item >= base + inc - ns && item < base + inc;
      const int L = __ffsll((unsigned long long)__ballot(mine)) - 1;
      b = b0 + L;
      split = item - base - __shfl(inc - ns, L, kWave);
      break;
    }
    base += total;
  }
  if (b < 0) return;
  const int nblk = blocks_of(ctx[b]);
  const int n = min(ctx[b], nblk * BS);
  const int blk_begin = split * chunk_blocks;
  const int blk_end = min(nblk, blk_begin + chunk_blocks);
  const int c = tid % LPT, tok0 = tid / LPT;

  // this thread's slice of the (pre-scaled) query of every head in the group
  float qf[G][VE], qs[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float tmp[VE];
    const T* qp = q + ((int64_t)b * Hq + g * G + h) * D + c * VE;
#pragma unroll
    for (int u = 0; u < VE / QE; ++u) unpack16(ld16(qp + u * QE), tmp + u * QE, T());
    qs[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      qf[h][e] = tmp[e] * scale_log2;
      qs[h] += qf[h][e];
    }
  }
  // m, l: running max and denominator; W: running sum of p * s_v (INT8 only)
  float m[G], l[G], W[G], o[G][VE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    W[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[h][e] = 0.f;
  }

  // physical ids of this split's blocks, one per lane (a split has at most
  // 64 blocks); invalid entries read block 0 instead of faulting
  const int nb = blk_end - blk_begin;
  int my_phys = 0;
  if (lane < nb) {
    const int p = bt[(int64_t)b * max_blocks + blk_begin + lane];
    my_phys = (p < 0 || p >= num_blocks) ? 0 : p;
  }
  // Loads are unconditional and two blocks deep: token slots past BS are
  // clamped into the block (their scores are masked), and past the split's
  // last block the loads repeat that block (cache hits, never used), so the
  // compiler's in-order load counting never has to drain the queue.
  // Slot s of the block: codes or values of row (phys, g, s); INT8 rows also
  // bring their K and V scales (ks, vs; unused otherwise).
  struct Buf {
    Ld k[NI], v[NI];
    float ks[NI], vs[NI];
  };
  auto gload = [&](Buf& r, int j) {
    const bool past = j >= nb;  // look-ahead past the split: one cached row
    const int phys = __builtin_amdgcn_readlane(my_phys, min(j, nb - 1));
    const int64_t srow = ((int64_t)phys * Hkv + g) * BS;
    const int64_t base = srow * D + c * VE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = past ? 0 : min(tok0 + i * TPI, BS - 1);
      r.k[i] = Sl::load(kc + base + (int64_t)tok * D);
      r.v[i] = Sl::load(vc + base + (int64_t)tok * D);
      if constexpr (Q8) {
        r.ks[i] = ksc[srow + tok];
        r.vs[i] = vsc[srow + tok];
      }
    }
  };
  auto process = [&](const Buf& r, int blk) {
    const int ntok = min(BS, n - blk * BS);
    float sc[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kv[VE];
      Sl::unpack(r.k[i], kv);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = Q8 ? -128.f * qs[h] : 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc += qf[h][e] * kv[e];
        sc[i][h] = acc;
      }
    }
    // reduce partial dots over the LPT lanes of each token
#pragma unroll
    for (int off = LPT / 2; off > 0; off >>= 1)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[i][h] += __shfl_xor(sc[i][h], off, kWave);
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[i][h] *= r.ks[i];
    }
    // mask, then the wave's online softmax over its tokens of this block
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tok = tok0 + i * TPI;
        if (!(tok < ntok)) sc[i][h] = -INFINITY;
        mx = fmaxf(mx, sc[i][h]);
      }
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
      const float m_new = fmaxf(m[h], mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m[h] - m_new);
      m[h] = m_new;
      l[h] *= alpha;
      W[h] *= alpha;
#pragma unroll
      for (int e = 0; e < VE; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pi = sc[i][h] == -INFINITY ? 0.f : exp2f(sc[i][h] - m_new);
        sc[i][h] = pi;
        l[h] += pi;     // per-lane partial; lanes of one token all add the same p
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = tok0 + i * TPI;
      if (tok < ntok) {
        float vv[VE];
        Sl::unpack(r.v[i], vv);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = Q8 ? sc[i][h] * r.vs[i] : sc[i][h];
          if constexpr (Q8) W[h] += w;
#pragma unroll
          for (int e = 0; e < VE; ++e) o[h][e] += w * vv[e];
        }
      }
    }
  };

  if constexpr (DEPTH >= 2) {
    // DEPTH blocks in flight, in whole groups: every iteration uses the
    // buffers in the order it refills them, so the loads in flight at the
    // loop head are the same on entry and on the back edge and no wait has
    // to drain them; the last group's refills (past the split: one cached
    // row) are never used
    Buf bufs[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) gload(bufs[u], u);
    int j = 0;
    for (; j + DEPTH <= nb; j += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        process(bufs[u], blk_begin + j + u);
        gload(bufs[u], j + u + DEPTH);
      }
    }
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u)
      if (j + u < nb) process(bufs[u], blk_begin + j + u);
  } else {
    // one block in flight (for query groups whose G x D of state per thread
    // leaves no registers for a second block)
    for (int j = 0; j < nb; ++j) {
      Buf ba;
      gload(ba, j);
      process(ba, blk_begin + j);
    }
  }
  if constexpr (Q8) {  // the -128 offset of the value codes
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VE; ++e) o[h][e] -= 128.f * W[h];
  }

  // merge the token lanes of each wave (fixed order), then the waves
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
      l[h] += __shfl_xor(l[h], off, kWave);
#pragma unroll
      for (int e = 0; e < VE; ++e) o[h][e] += __shfl_xor(o[h][e], off, kWave);
    }
  }
  // lanes 0 .. LPT-1 now hold the wave's o slices; every lane of a token
  // group carried the same l, so lane 0's value is the wave's sum
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (c == 0) {
        red_m[wave][h] = m[h];
        red_l[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) red_o[wave][h][c * VE + e] = o[h][e];
    }
  }
  __syncthreads();
  const int64_t row0 = ((int64_t)b * Hq + g * G) * max_splits + split;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, red_m[w][h]);
    float oa = 0.f, la = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float sw = red_m[w][h] == -INFINITY ? 0.f : exp2f(red_m[w][h] - M);
      oa += sw * red_o[w][h][d];
      la += sw * red_l[w][h];
    }
    float* dst = ws + (row0 + (int64_t)h * max_splits) * (D + 2);
    dst[d] = oa;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = la;
    }
  }
}

// Combine the splits of one (sequence, head) in fixed order.
template <typename T, int D>
__global__ void __launch_bounds__(kCombineThreads)
attn_decode_combine(const float* __restrict__ ws, const int32_t* __restrict__ ctx,
                    T* __restrict__ out, int Hq, int BS, int chunk_blocks, int max_splits) {
  const int b = blockIdx.y, h = blockIdx.x;
  const int nblk = (ctx[b] + BS - 1) / BS;
  const int ns = min((nblk + chunk_blocks - 1) / chunk_blocks, max_splits);
  combine_row<T, D>(ws + ((int64_t)b * Hq + h) * max_splits * (D + 2), ns,
                    out + ((int64_t)b * Hq + h) * D);
}

// Slice size and pipeline depth.  Layer-dtype caches: 16-byte slices, two
// blocks in flight.  INT8: 16-byte slices (16 codes) for query groups of up
// to two heads, measured 5.4 TB/s on the 7B decode shape against 4.7-5.3 TB/s
// for 8-byte slices, whose blocks carry half the bytes per load; deeper
// pipelines (3, 4 blocks) gained nothing.  Larger groups keep 8-byte slices
// and one block in flight, since every thread holds G x VE query and output
// values (a second block spilled registers at G 8 and ran slower at G 4).
template <typename KV, int G>
struct DecTune {
  static constexpr int SB = 16, DEPTH = G <= 2 ? 2 : 1;
};
template <int G>
struct DecTune<int8_t, G> {
  static constexpr int SB = G <= 2 ? 16 : 8, DEPTH = G <= 2 ? 2 : 1;
};

template <typename T, typename KV, int D, int G>
static hipError_t launch_dec(const T* q, const KV* kc, const KV* vc, const float* ks,
                             const float* vs, const int32_t* bt, int max_blocks,
                             const int32_t* ctx, int B, int Hq, int Hkv, int BS, float sl2,
                             const DecodePlan& pl, float* ws, int num_blocks, hipStream_t st) {
  const dim3 grid(pl.max_splits * Hkv * B);
  constexpr int SB = DecTune<KV, G>::SB, DEPTH = DecTune<KV, G>::DEPTH;
  hipLaunchKernelGGL((attn_decode_kernel<T, KV, D, G, SB, DEPTH>), grid,
                     dim3(kDecThreads), 0, st, q, kc,
                     vc, ks, vs, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl.chunk_blocks,
                     pl.max_splits, ws, num_blocks);
  return hipGetLastError();
}

template <typename T, typename KV, int D>
static hipError_t dispatch_g(const T* q, const KV* kc, const KV* vc, const float* ks,
                             const float* vs, const int32_t* bt, int max_blocks,
                             const int32_t* ctx, int B, int Hq, int Hkv, int BS, float sl2,
                             const DecodePlan& pl, float* ws, int num_blocks, hipStream_t st) {
  switch (Hq / Hkv) {
    case 1: return launch_dec<T, KV, D, 1>(q, kc, vc, ks, vs, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 2: return launch_dec<T, KV, D, 2>(q, kc, vc, ks, vs, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 4: return launch_dec<T, KV, D, 4>(q, kc, vc, ks, vs, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 8: return launch_dec<T, KV, D, 8>(q, kc, vc, ks, vs, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename KV>
static hipError_t decode_impl(const T* q, const KV* k_cache, const KV* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                              float scale, T* out, const DecodePlan& pl, void* ws, int num_blocks,
                              hipStream_t st) {
  if (B == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  float* w = reinterpret_cast<float*>(ws);
  hipError_t e;
  if (D == 128)
    e = dispatch_g<T, KV, 128>(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks,
                               context_lens, B, Hq, Hkv, BS, sl2, pl, w, num_blocks, st);
  else if (D == 64)
    e = dispatch_g<T, KV, 64>(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks,
                              context_lens, B, Hq, Hkv, BS, sl2, pl, w, num_blocks, st);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  if (D == 128)
    hipLaunchKernelGGL((attn_decode_combine<T, 128>), dim3(Hq, B), dim3(kCombineThreads), 0, st, w,
                       context_lens, out, Hq, BS, pl.chunk_blocks, pl.max_splits);
  else
    hipLaunchKernelGGL((attn_decode_combine<T, 64>), dim3(Hq, B), dim3(kCombineThreads), 0, st, w,
                       context_lens, out, Hq, BS, pl.chunk_blocks, pl.max_splits);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_decode_paged(const T* q, const T* k_cache, const T* v_cache,
                             const int32_t* block_table, int max_blocks,
                             const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                             float scale, T* out, const DecodePlan& pl, void* ws, int num_blocks,
                             hipStream_t st) {
  if (pl.narrow_ck > 0)
    return attn_decode_narrow<T>(q, k_cache, v_cache, block_table, max_blocks, context_lens, B, Hq,
                                 Hkv, D, BS, pl.narrow_sp * pl.narrow_ck, scale, out,
                                 pl.narrow_ck, pl.narrow_sp, ws, num_blocks, st);
  return decode_impl<T, T>(q, k_cache, v_cache, nullptr, nullptr, block_table, max_blocks,
                           context_lens, B, Hq, Hkv, D, BS, scale, out, pl, ws, num_blocks, st);
}

template <typename T>
hipError_t attn_decode_paged_q8(const T* q, const int8_t* k_codes, const int8_t* v_codes,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int max_blocks,
                                const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                                int BS, float scale, T* out, const DecodePlan& pl, void* ws,
                                int num_blocks, hipStream_t st) {
  return decode_impl<T, int8_t>(q, k_codes, v_codes, k_scale, v_scale, block_table, max_blocks,
                                context_lens, B, Hq, Hkv, D, BS, scale, out, pl, ws, num_blocks,
                                st);
}

template hipError_t attn_decode_paged<bf16>(const bf16*, const bf16*, const bf16*, const int32_t*,
                                            int, const int32_t*, int, int, int, int, int, float,
                                            bf16*, const DecodePlan&, void*, int, hipStream_t);
template hipError_t attn_decode_paged<float>(const float*, const float*, const float*,
                                             const int32_t*, int, const int32_t*, int, int, int,
                                             int, int, float, float*, const DecodePlan&, void*,
                                             int, hipStream_t);
template hipError_t attn_decode_paged_q8<bf16>(const bf16*, const int8_t*, const int8_t*,
                                               const float*, const float*, const int32_t*, int,
                                               const int32_t*, int, int, int, int, int, float,
                                               bf16*, const DecodePlan&, void*, int, hipStream_t);
template hipError_t attn_decode_paged_q8<float>(const float*, const int8_t*, const int8_t*,
                                                const float*, const float*, const int32_t*, int,
                                                const int32_t*, int, int, int, int, int, float,
                                                float*, const DecodePlan&, void*, int,
                                                hipStream_t);

}  // namespace dl
