// unfused.hip -- the kernel-per-op chain of a decoder layer before fusion.
//
// The ops-transformer Llama2-7B page ("single-layer operator call chain")
// lists the layer as separate kernels before fusion: Q, K and V linears, a
// rotary-embedding kernel, Q.K^T, softmax and .V as three kernels, the output
// linear, then the FFN as gate linear, up linear, SiLU, the gate x up product
// and the down linear, plus norms and residual adds.  Every intermediate
// round-trips HBM.  These kernels implement that chain (simple SIMT code; the
// projections reuse the MFMA GEMM without epilogue fusion) so the fused path
// can be compared against it in time and in HBM bytes.  The score matrix is
// written in fp32 and the probabilities in the activation dtype.
#include "dl_internal.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// RoPE as its own pass (rotate-half, table [max_pos][D/2][2])
// ---------------------------------------------------------------------------
template <typename T>
__global__ void unf_rope_kernel(T* __restrict__ u, const int32_t* __restrict__ pos,
                                const float* __restrict__ cs, int max_pos, int T_, int nh, int D) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T_ * nh * half;
  if (idx >= total) return;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;
  const int t = (int)(th / nh);
  T* row = u + th * D;
  const int p = min(max(pos[t], 0), max_pos - 1);
  const float c = cs[((int64_t)p * half + i) * 2], s = cs[((int64_t)p * half + i) * 2 + 1];
  const float a = to_f32(row[i]), b = to_f32(row[i + half]);
  row[i] = from_f32<T>(a * c - b * s);
  row[i + half] = from_f32<T>(b * c + a * s);
}

template <typename T>
hipError_t unf_rope(T* u, const int32_t* pos, const float* cs, int max_pos, int T_, int nh, int D,
                    hipStream_t st) {
  const int64_t n = (int64_t)T_ * nh * (D / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_rope_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, u,
                     pos, cs, max_pos, T_, nh, D);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill scores: S[b][h][i][j] = scale * q_i . k_j (j <= i), -inf otherwise,
// for i, j < S_b; row stride S_max.  64x64 tile per workgroup, 4x4 per thread.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
unf_scores_kernel(const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ cu,
                  int S_max, int Hq, int Hkv, int D, float scale, float* __restrict__ S) {
  __shared__ float Qs[64][33], Ks[64][33];
  const int b = blockIdx.z, h = blockIdx.y;
  const int tiles_j = (S_max + 63) / 64;
  const int ti = blockIdx.x / tiles_j, tj = blockIdx.x % tiles_j;
  const int t0 = cu[b], Sb = min(cu[b + 1] - t0, S_max);
  if (ti * 64 >= Sb || tj * 64 >= Sb) return;
  const int g = h / (Hq / Hkv);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += 32) {
    for (int e = threadIdx.x; e < 64 * 32; e += 256) {
      const int r = e / 32, c = e % 32;
      const int qi = ti * 64 + r, kj = tj * 64 + r;
      Qs[r][c] = qi < Sb ? to_f32(q[((int64_t)(t0 + qi) * Hq + h) * D + d0 + c]) : 0.f;
      Ks[r][c] = kj < Sb ? to_f32(k[((int64_t)(t0 + kj) * Hkv + g) * D + d0 + c]) : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < 32; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) acc[a][bb] += Qs[ty * 4 + a][c] * Ks[tx * 4 + bb][c];
    __syncthreads();
  }
  float* base = S + (((int64_t)b * Hq + h) * S_max) * S_max;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int i = ti * 64 + ty * 4 + a, j = tj * 64 + tx * 4 + bb;
      if (i < Sb && j < Sb) base[(int64_t)i * S_max + j] = j <= i ? acc[a][bb] * scale : -INFINITY;
    }
}

template <typename T>
hipError_t unf_scores(const T* q, const T* k, const int32_t* cu, int B, int S_max, int Hq,
                      int Hkv, int D, float scale, float* S, hipStream_t st) {
  if (B == 0 || S_max == 0) return hipSuccess;
  const int tiles = (S_max + 63) / 64;
  hipLaunchKernelGGL((unf_scores_kernel<T>), dim3(tiles * tiles, Hq, B), dim3(256), 0, st, q, k,
                     cu, S_max, Hq, Hkv, D, scale, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax over rows of S (one wave per row) -> P in the activation dtype.
// Prefill: row (b, h, i), length S_b.  Decode: row (b, h), length ctx_b.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64)
unf_softmax_kernel(const float* __restrict__ S, T* __restrict__ P, const int32_t* __restrict__ lens,
                   int lens_are_cu, int S_max, int Hq, int rows_per_head) {
  // Rows of up to 64 x kHeld floats are read once and kept in registers;
  // longer rows take an online (max, sum) pass and a write pass.
  constexpr int kHeld = 64;
  const int b = blockIdx.z, h = blockIdx.y, i = blockIdx.x;
  const int n = min(lens_are_cu ? lens[b + 1] - lens[b] : lens[b], S_max);
  if (rows_per_head > 1 && i >= n) return;
  const int64_t row = (((int64_t)b * Hq + h) * rows_per_head + i) * S_max;
  const int lane = threadIdx.x;
  if (n <= 64 * kHeld) {
    float v[kHeld];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kHeld; ++e) {
      const int j = lane + 64 * e;
      v[e] = j < n ? S[row + j] : -INFINITY;
      mx = fmaxf(mx, v[e]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < kHeld; ++e) {
      v[e] = __expf(v[e] - mx);
      sum += v[e];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < kHeld; ++e) {
      const int j = lane + 64 * e;
      if (j < n) P[row + j] = from_f32<T>(v[e] * inv);
    }
    return;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float x = S[row + j];
    const float mn = fmaxf(m, x);
    l = l * __expf(m - mn) + __expf(x - mn);
    m = mn;
  }
  const float M = wave_max(m);
  const float L = wave_sum(m == -INFINITY ? 0.f : l * __expf(m - M));
  const float inv = 1.0f / L;
  for (int j = lane; j < n; j += 64) P[row + j] = from_f32<T>(__expf(S[row + j] - M) * inv);
}

template <typename T>
hipError_t unf_softmax(const float* S, T* P, const int32_t* lens, bool lens_are_cu, int B,
                       int S_max, int Hq, int rows_per_head, hipStream_t st) {
  if (B == 0 || S_max == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_softmax_kernel<T>), dim3(rows_per_head, Hq, B), dim3(64), 0, st, S, P,
                     lens, lens_are_cu ? 1 : 0, S_max, Hq, rows_per_head);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill PV: out[t0+i][h][:] = sum_j P[b][h][i][j] v[t0+j][g][:].
// 64 rows x D columns per workgroup; thread owns 4 rows x (D/16) columns.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
unf_pv_kernel(const T* __restrict__ P, const T* __restrict__ v, const int32_t* __restrict__ cu,
              int S_max, int Hq, int Hkv, int D, T* __restrict__ out) {
  __shared__ float Ps[64][33];
  __shared__ float Vs[32][129];
  const int b = blockIdx.z, h = blockIdx.y, ti = blockIdx.x;
  const int t0 = cu[b], Sb = min(cu[b + 1] - t0, S_max);
  if (ti * 64 >= Sb) return;
  const int g = h / (Hq / Hkv);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int CPT = D / 16;  // columns per thread (4 or 8)
  float acc[4][8] = {};
  const T* prow = P + (((int64_t)b * Hq + h) * S_max) * S_max;
  for (int j0 = 0; j0 < Sb; j0 += 32) {
    for (int e = threadIdx.x; e < 64 * 32; e += 256) {
      const int r = e / 32, c = e % 32;
      const int i = ti * 64 + r, j = j0 + c;
      Ps[r][c] = (i < Sb && j < Sb) ? to_f32(prow[(int64_t)i * S_max + j]) : 0.f;
    }
    for (int e = threadIdx.x; e < 32 * D; e += 256) {
      const int r = e / D, c = e % D;
      const int j = j0 + r;
      Vs[r][c] = j < Sb ? to_f32(v[((int64_t)(t0 + j) * Hkv + g) * D + c]) : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < 32; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
          if (bb < CPT) acc[a][bb] += Ps[ty * 4 + a][c] * Vs[c][tx * CPT + bb];
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = ti * 64 + ty * 4 + a;
    if (i < Sb)
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        if (bb < CPT)
          out[((int64_t)(t0 + i) * Hq + h) * D + tx * CPT + bb] = from_f32<T>(acc[a][bb]);
  }
}

template <typename T>
hipError_t unf_pv(const T* P, const T* v, const int32_t* cu, int B, int S_max, int Hq, int Hkv,
                  int D, T* out, hipStream_t st) {
  if (B == 0 || S_max == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_pv_kernel<T>), dim3((S_max + 63) / 64, Hq, B), dim3(256), 0, st, P, v,
                     cu, S_max, Hq, Hkv, D, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode, reading the paged cache directly: scores S[b][h][j] (stride
// ctx_max) and PV.  One workgroup per (b, h).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256)
unf_dec_scores_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                      const int32_t* __restrict__ bt, int max_blocks,
                      const int32_t* __restrict__ ctx, int ctx_max, int Hq, int Hkv, int D,
                      int BS, float scale, float* __restrict__ S, int num_blocks) {
  __shared__ float qs[128];
  const int b = blockIdx.y, h = blockIdx.x, g = h / (Hq / Hkv);
  for (int d = threadIdx.x; d < D; d += 256) qs[d] = to_f32(q[((int64_t)b * Hq + h) * D + d]);
  __syncthreads();
  const int n = min(min(ctx[b], ctx_max), max_blocks * BS);
  for (int j = threadIdx.x; j < n; j += 256) {
    int phys = bt[(int64_t)b * max_blocks + j / BS];
    phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;
    const T* kr = kc + (((int64_t)phys * Hkv + g) * BS + j % BS) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += qs[d] * to_f32(kr[d]);
    S[((int64_t)b * Hq + h) * ctx_max + j] = acc * scale;
  }
}

template <typename T>
__global__ void __launch_bounds__(128)
unf_dec_pv_kernel(const T* __restrict__ P, const T* __restrict__ vc, const int32_t* __restrict__ bt,
                  int max_blocks, const int32_t* __restrict__ ctx, int ctx_max, int Hq, int Hkv,
                  int D, int BS, T* __restrict__ out, int num_blocks) {
  const int b = blockIdx.y, h = blockIdx.x, g = h / (Hq / Hkv), d = threadIdx.x;
  if (d >= D) return;
  const int n = min(min(ctx[b], ctx_max), max_blocks * BS);
  const T* prow = P + ((int64_t)b * Hq + h) * ctx_max;
  float acc = 0.f;
  for (int j = 0; j < n; ++j) {
    int phys = bt[(int64_t)b * max_blocks + j / BS];
    phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;
    acc += to_f32(prow[j]) * to_f32(vc[(((int64_t)phys * Hkv + g) * BS + j % BS) * D + d]);
  }
  out[((int64_t)b * Hq + h) * D + d] = from_f32<T>(acc);
}

template <typename T>
hipError_t unf_dec_attn(const T* q, const T* kc, const T* vc, const int32_t* bt, int max_blocks,
                        const int32_t* ctx, int ctx_max, int B, int Hq, int Hkv, int D, int BS,
                        float scale, float* S, T* P, T* out, int num_blocks, hipStream_t st) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_dec_scores_kernel<T>), dim3(Hq, B), dim3(256), 0, st, q, kc, bt,
                     max_blocks, ctx, ctx_max, Hq, Hkv, D, BS, scale, S, num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = unf_softmax<T>(S, P, ctx, false, B, ctx_max, Hq, 1, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((unf_dec_pv_kernel<T>), dim3(Hq, B), dim3(128), 0, st, P, vc, bt, max_blocks,
                     ctx, ctx_max, Hq, Hkv, D, BS, out, num_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// elementwise
// ---------------------------------------------------------------------------
template <typename T>
__global__ void unf_add_kernel(const float* __restrict__ a, const T* __restrict__ b,
                               float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = a[i] + to_f32(b[i]);
}
template <typename T>
__global__ void unf_silu_kernel(const T* __restrict__ g, T* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = from_f32<T>(silu(to_f32(g[i])));
}
template <typename T>
__global__ void unf_mul_kernel(const T* __restrict__ a, const T* __restrict__ b,
                               T* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = from_f32<T>(to_f32(a[i]) * to_f32(b[i]));
}

static inline dim3 grid1(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

template <typename T>
hipError_t unf_add(const float* a, const T* b, float* out, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_add_kernel<T>), grid1(n), dim3(256), 0, st, a, b, out, n);
  return hipGetLastError();
}
template <typename T>
hipError_t unf_silu(const T* g, T* out, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_silu_kernel<T>), grid1(n), dim3(256), 0, st, g, out, n);
  return hipGetLastError();
}
template <typename T>
hipError_t unf_mul(const T* a, const T* b, T* out, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((unf_mul_kernel<T>), grid1(n), dim3(256), 0, st, a, b, out, n);
  return hipGetLastError();
}

#define DL_UNF_INST(T)                                                                          \
  template hipError_t unf_rope<T>(T*, const int32_t*, const float*, int, int, int, int,         \
                                  hipStream_t);                                                 \
  template hipError_t unf_scores<T>(const T*, const T*, const int32_t*, int, int, int, int, int, \
                                    float, float*, hipStream_t);                                \
  template hipError_t unf_softmax<T>(const float*, T*, const int32_t*, bool, int, int, int, int, \
                                     hipStream_t);                                              \
  template hipError_t unf_pv<T>(const T*, const T*, const int32_t*, int, int, int, int, int, T*, \
                                hipStream_t);                                                   \
  template hipError_t unf_dec_attn<T>(const T*, const T*, const T*, const int32_t*, int,        \
                                      const int32_t*, int, int, int, int, int, int, float,       \
                                      float*, T*, T*, int, hipStream_t);                        \
  template hipError_t unf_add<T>(const float*, const T*, float*, int64_t, hipStream_t);         \
  template hipError_t unf_silu<T>(const T*, T*, int64_t, hipStream_t);                          \
  template hipError_t unf_mul<T>(const T*, const T*, T*, int64_t, hipStream_t);

DL_UNF_INST(bf16)
DL_UNF_INST(float)

}  // namespace dl
