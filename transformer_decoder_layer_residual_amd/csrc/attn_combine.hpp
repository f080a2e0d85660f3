// attn_combine.hpp -- merge of split-KV attention partials (gfx950).
//
// A split s of one (query row, head) leaves o_s[D] = sum_j exp2(x_j - m_s) v_j,
// m_s = max_j x_j and l_s = sum_j exp2(x_j - m_s) over its keys (log2-domain
// scores x_j).  The row's attention output is
//   sum_s w_s o_s / sum_s w_s l_s,  w_s = exp2(m_s - M),  M = max_s m_s
// (the rescaling of the online softmax in the flash-attention page, applied
// once over the splits).  Splits with no keys carry m_s = -inf and weigh 0; a
// row with no keys at all gets 0.
//
// One 256-thread workgroup per row, arranged as a D x P grid (P = 256 / D).
// All loads of the common case go out together before any is used: thread
// s reads (m_s, l_s) of split s, and thread (d, p) reads o_s[d] of its first
// eight splits s = p, p + P, ...  The block reduces M; thread s puts w_s and
// w_s l_s into LDS; thread (d, p) adds w_s o_s[d] over its splits in order
// (loading the rest, beyond 256 splits or its first eight, as it goes) and
// the P partial sums are added in fixed order, so the result does not depend
// on timing.  (One thread per d walking the splits with one load at a time
// took 18 us for 32 splits of 64 heads; three dependent load phases took
// 16 us for 8192 one-split rows.)
#pragma once

#include "dl_common.hpp"

namespace dl {

constexpr int kCombineThreads = 256;

template <typename T, int D>
__device__ __forceinline__ void combine_row(const float* __restrict__ base, int ns,
                                            T* __restrict__ dst) {
  constexpr int NT = kCombineThreads, P = NT / D, W = NT / kWave, PF = 8;
  static_assert(P * D == NT, "D divides the workgroup");
  __shared__ float w_s[NT], wl_s[NT], red[W];
  __shared__ float part[P][D + 1];
  const int tid = threadIdx.x, d = tid % D, pr = tid / D;
  if (ns <= 0) {  // no keys: the row is 0
    if (pr == 0) dst[d] = from_f32<T>(0.f);
    return;
  }
  const int64_t RS = D + 2;  // floats per split record
  // ---- every load of the first chunk at once (indices clamped to ns - 1)
  const float* own = base + (int64_t)min(tid, ns - 1) * RS;
  const float m_own = own[D], l_own = own[D + 1];
  float ov[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) ov[k] = base[(int64_t)min(pr + k * P, ns - 1) * RS + d];

  float m = tid < ns ? m_own : -INFINITY;
  for (int s = tid + NT; s < ns; s += NT) m = fmaxf(m, base[(int64_t)s * RS + D]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) M = fmaxf(M, red[w]);

  float num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < ns; c0 += NT) {
    const int s = c0 + tid;
    float w = 0.f, wl = 0.f;
    if (s < ns) {
      float ms = m_own, ls = l_own;
      if (c0 > 0) {
        const float* ps = base + (int64_t)s * RS;
        ms = ps[D];
        ls = ps[D + 1];
      }
      w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      wl = w * ls;
    }
    w_s[tid] = w;
    wl_s[tid] = wl;
    __syncthreads();
    const int n = min(NT, ns - c0);
    int j = pr;
    if (c0 == 0) {
#pragma unroll
      for (int k = 0; k < PF; ++k, j += P)
        if (j < n) {
          num += w_s[j] * ov[k];
          den += wl_s[j];
        }
    }
    const float* pc = base + (int64_t)c0 * RS + d;
#pragma unroll 8
    for (; j < n; j += P) {
      num += w_s[j] * pc[(int64_t)j * RS];
      den += wl_s[j];
    }
    __syncthreads();  // w_s, wl_s reused by the next chunk
  }
  if constexpr (P > 1) {
    part[pr][d] = num;
    if (d == 0) part[pr][D] = den;
    __syncthreads();
    if (pr == 0) {
      num = part[0][d];
      den = part[0][D];
#pragma unroll
      for (int p = 1; p < P; ++p) {
        num += part[p][d];
        den += part[p][D];
      }
    }
  }
  if (pr == 0) dst[d] = from_f32<T>(den > 0.f ? num / den : 0.f);
}

}  // namespace dl
