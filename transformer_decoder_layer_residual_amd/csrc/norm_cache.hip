// norm_cache.hip -- RMSNorm (optionally fused with the residual add), the
// RoPE cos/sin table, and reshape-and-cache into paged KV blocks.
#include "dl_internal.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// RMSNorm + residual.  One workgroup per token row; the row stays in
// registers between the statistics pass and the scaling pass, so x (and the
// residual) are read once and h / out written once.
//   resid_in == nullptr:  out = gamma * x / sqrt(mean(x^2) + eps)
//   otherwise:            h = x + resid_in (fp32) -> resid_out,
//                         out = gamma * h / sqrt(mean(h^2) + eps)
// (Llama RMSNorm in the layer chain of the ops-transformer Llama2-7B page;
// norm fused with the residual add per the "fusion operator matrix" section of
// the ascend-transformer-boost page.)
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 256;
constexpr int kNormMaxVec = 8;  // 4-element vectors per thread: H <= 8192

template <typename T>
__device__ __forceinline__ f32x4 ld4f(const T* p) {
  float o[4];
  load4(p, o);
  return f32x4{o[0], o[1], o[2], o[3]};
}

// NV: 4-element vectors per thread (H <= 4 * NV * NT).  NT = 256 threads per
// row for prefill-sized row counts; 1024 for a handful of decode rows, where
// the few workgroups' load latency, not bandwidth, sets the time.
template <typename Tin, typename Tout, int NV, int NT = kNormThreads>
__global__ void __launch_bounds__(NT)
rmsnorm_kernel(const Tin* __restrict__ x, const float* __restrict__ rin, float* __restrict__ rout,
               const Tout* __restrict__ gamma, Tout* __restrict__ out, int H, float eps) {
  constexpr int kNormThreads = NT;
  __shared__ float red[kNormThreads / kWave];
  const int64_t row = blockIdx.x;
  const int nv = H / 4;
  const int tid = threadIdx.x;
  // Every load is issued before the first use (indices clamped into the
  // row, results of the clamped lanes unused): with the loads under the
  // per-vector bounds test the compiler waited for each one in turn.
  f32x4 h[NV], g[NV], rr[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = min(tid + i * kNormThreads, nv - 1);
    h[i] = ld4f(x + row * H + 4 * v);
    g[i] = ld4f(gamma + 4 * v);
    if (rin) rr[i] = *reinterpret_cast<const f32x4*>(rin + row * H + 4 * v);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kNormThreads;
    if (v < nv) {
      if (rin) {
        h[i] = h[i] + rr[i];
        *reinterpret_cast<f32x4*>(rout + row * H + 4 * v) = h[i];
      }
      ss += h[i][0] * h[i][0] + h[i][1] * h[i][1] + h[i][2] * h[i][2] + h[i][3] * h[i][3];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kNormThreads;
    if (v < nv)
      store4(out + row * H + 4 * v, g[i][0] * (h[i][0] * inv), g[i][1] * (h[i][1] * inv),
             g[i][2] * (h[i][2] * inv), g[i][3] * (h[i][3] * inv));
  }
}

template <typename Tin, typename Tout>
hipError_t rmsnorm_residual(const Tin* x, const float* resid_in, float* resid_out,
                            const Tout* gamma, Tout* out, int T, int H, float eps,
                            hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (T <= 64 && H / 4 > 2 * kNormThreads) {
    // decode-sized: 1024 threads per row, at most 2 vectors each (H <= 8192)
    if (H / 4 <= 1024)
      hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, 1, 1024>), dim3(T), dim3(1024), 0, st, x,
                         resid_in, resid_out, gamma, out, H, eps);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, 2, 1024>), dim3(T), dim3(1024), 0, st, x,
                         resid_in, resid_out, gamma, out, H, eps);
    return hipGetLastError();
  }
  const int nvt = (H / 4 + kNormThreads - 1) / kNormThreads;
  if (nvt <= 1)
    hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, 1>), dim3(T), dim3(kNormThreads), 0, st, x,
                       resid_in, resid_out, gamma, out, H, eps);
  else if (nvt <= 2)
    hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, 2>), dim3(T), dim3(kNormThreads), 0, st, x,
                       resid_in, resid_out, gamma, out, H, eps);
  else if (nvt <= 4)
    hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, 4>), dim3(T), dim3(kNormThreads), 0, st, x,
                       resid_in, resid_out, gamma, out, H, eps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<Tin, Tout, kNormMaxVec>), dim3(T), dim3(kNormThreads), 0,
                       st, x, resid_in, resid_out, gamma, out, H, eps);
  return hipGetLastError();
}

template hipError_t rmsnorm_residual<float, bf16>(const float*, const float*, float*, const bf16*,
                                                  bf16*, int, int, float, hipStream_t);
template hipError_t rmsnorm_residual<bf16, bf16>(const bf16*, const float*, float*, const bf16*,
                                                 bf16*, int, int, float, hipStream_t);
template hipError_t rmsnorm_residual<float, float>(const float*, const float*, float*,
                                                   const float*, float*, int, int, float,
                                                   hipStream_t);
template hipError_t rmsnorm_residual<bf16, float>(const bf16*, const float*, float*, const float*,
                                                  float*, int, int, float, hipStream_t);

// ---------------------------------------------------------------------------
// RoPE table: cos_sin[p][i] = (cos, sin)(p * theta^(-2i/D)), angle in fp64.
// (Rotate-half pairing; the pages name the rotary embedding but print no
// formula, so the common Llama form is taken.)
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float* cs, int max_pos, int half, int D, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double w = pow(theta, -2.0 * (double)i / (double)D);
  const double phi = (double)p * w;
  cs[2 * idx] = (float)cos(phi);
  cs[2 * idx + 1] = (float)sin(phi);
}

hipError_t rope_table_fill(float* cs, int max_pos, int D, double theta, hipStream_t st) {
  const int half = D / 2;
  const int64_t n = (int64_t)max_pos * half;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cs,
                     max_pos, half, D, theta);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reshape-and-cache: token t (sequence s, position p) of kv head g goes to
// block block_table[s][p / BS], slot p % BS of the [num_blocks][Hkv][BS][D]
// cache (ATB KV-cache page, "KV cache memory bottleneck": paged blocks
// addressed through block_table, ReshapeAndCache writing step K/V).
// One thread per 16-byte vector; a pure copy, so the result is bit-exact.
// Out-of-range table entries are skipped (the write is dropped) instead of
// faulting.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void reshape_and_cache_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                         const int32_t* __restrict__ seq_of_token,
                                         const int32_t* __restrict__ pos,
                                         const int32_t* __restrict__ block_table, int max_blocks,
                                         T* __restrict__ kc, T* __restrict__ vc, int T_, int Hkv,
                                         int D, int BS, int num_blocks) {
  constexpr int VE = 16 / sizeof(T);
  const int vpr = D / VE;  // vectors per head row
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T_ * Hkv * vpr;
  if (idx >= total) return;
  const int c = (int)(idx % vpr);
  const int64_t tg = idx / vpr;
  const int g = (int)(tg % Hkv);
  const int t = (int)(tg / Hkv);
  const int s = seq_of_token ? seq_of_token[t] : t, p = pos[t];
  if (p < 0 || p / BS >= max_blocks) return;
  const int blk = block_table[(int64_t)s * max_blocks + p / BS];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t dst = (((int64_t)blk * Hkv + g) * BS + (p % BS)) * D + c * VE;
  const int64_t src = ((int64_t)t * Hkv + g) * D + c * VE;
  st16(kc + dst, ld16(k + src));
  st16(vc + dst, ld16(v + src));
}

template <typename T>
hipError_t reshape_and_cache(const T* k, const T* v, const int32_t* seq_of_token,
                             const int32_t* pos, const int32_t* block_table, int max_blocks,
                             T* k_cache, T* v_cache, int T_, int Hkv, int D, int BS,
                             int num_blocks, hipStream_t st) {
  const int64_t n = (int64_t)T_ * Hkv * (D / (16 / (int)sizeof(T)));
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((reshape_and_cache_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                     0, st, k, v, seq_of_token, pos, block_table, max_blocks, k_cache, v_cache,
                     T_, Hkv, D, BS, num_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reshape-and-cache into an INT8 cache, quantising each row on the way in
// (ATB KV-cache page, section "KV cache quantisation": per-token granularity,
// one fp32 scale for a token's K and one for its V, computed online when the
// token is written).  A row is one (token, kv head) D-vector of K or of V:
//   scale = max|x| / 127, code = x / scale rounded half to even, clamped to
//   [-127, 127], both in fp32; an all-zero row gets scale 0 and zero codes.
// Codes land where reshape_and_cache would put the values; the scale of a row
// sits at the same (block, head, slot) of a [num_blocks][Hkv][BS] fp32 array.
// One group of D / VE lanes (one 16-byte slice each) per (token, kv head);
// the group's absolute maximum is reduced with lane shuffles.  A group is
// never split across waves (64 is a multiple of D / VE), and every lane of a
// group shares its row, so the shuffles only ever pair lanes of one row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quant4(const float* x, float s) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r = 0.f;
    if (s != 0.f) r = fminf(fmaxf(rintf(x[e] / s), -127.f), 127.f);
    w |= ((uint32_t)(int32_t)r & 0xffu) << (8 * e);
  }
  return w;
}

template <typename T>
__device__ __forceinline__ void quant_slice(const T* src, int lpr, int8_t* dst, float* sdst,
                                            bool lead) {
  constexpr int VE = 16 / sizeof(T);
  float x[VE];
  unpack16(ld16(src), x, T());
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < VE; ++e) amax = fmaxf(amax, fabsf(x[e]));
  for (int off = 1; off < lpr; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const float s = amax / 127.0f;
  if (!dst) return;
  if constexpr (VE == 8) {
    u32x2 w = {quant4(x, s), quant4(x + 4, s)};
    *reinterpret_cast<u32x2*>(dst) = w;
  } else {
    *reinterpret_cast<uint32_t*>(dst) = quant4(x, s);
  }
  if (lead) *sdst = s;
}

template <typename T>
__global__ void reshape_and_cache_q8_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                            const int32_t* __restrict__ seq_of_token,
                                            const int32_t* __restrict__ pos,
                                            const int32_t* __restrict__ block_table,
                                            int max_blocks, int8_t* __restrict__ kq,
                                            int8_t* __restrict__ vq, float* __restrict__ ks,
                                            float* __restrict__ vs, int T_, int Hkv, int D, int BS,
                                            int num_blocks) {
  constexpr int VE = 16 / sizeof(T);
  const int lpr = D / VE;  // lanes per row, a power of two dividing 64
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)T_ * Hkv;
  const int64_t row = min(idx / lpr, rows - 1);  // the grid's tail repeats the last row
  const int c = (int)(idx % lpr);
  const int g = (int)(row % Hkv);
  const int t = (int)(row / Hkv);
  const int s = seq_of_token ? seq_of_token[t] : t, p = pos[t];
  bool keep = idx / lpr < rows && p >= 0 && p / BS < max_blocks;
  int blk = 0;
  if (keep) {
    blk = block_table[(int64_t)s * max_blocks + p / BS];
    keep = blk >= 0 && blk < num_blocks;
  }
  const int64_t drow = ((int64_t)blk * Hkv + g) * BS + (p % BS);
  const int64_t src = ((int64_t)t * Hkv + g) * D + c * VE;
  quant_slice(k + src, lpr, keep ? kq + drow * D + c * VE : nullptr, ks + drow, c == 0);
  quant_slice(v + src, lpr, keep ? vq + drow * D + c * VE : nullptr, vs + drow, c == 0);
}

template <typename T>
hipError_t reshape_and_cache_q8(const T* k, const T* v, const int32_t* seq_of_token,
                                const int32_t* pos, const int32_t* block_table, int max_blocks,
                                int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                                int T_, int Hkv, int D, int BS, int num_blocks, hipStream_t st) {
  const int64_t n = (int64_t)T_ * Hkv * (D / (16 / (int)sizeof(T)));
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((reshape_and_cache_q8_kernel<T>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, st, k, v, seq_of_token, pos, block_table, max_blocks, k_codes,
                     v_codes, k_scale, v_scale, T_, Hkv, D, BS, num_blocks);
  return hipGetLastError();
}

template hipError_t reshape_and_cache_q8<bf16>(const bf16*, const bf16*, const int32_t*,
                                               const int32_t*, const int32_t*, int, int8_t*,
                                               int8_t*, float*, float*, int, int, int, int, int,
                                               hipStream_t);
template hipError_t reshape_and_cache_q8<float>(const float*, const float*, const int32_t*,
                                                const int32_t*, const int32_t*, int, int8_t*,
                                                int8_t*, float*, float*, int, int, int, int, int,
                                                hipStream_t);

template hipError_t reshape_and_cache<bf16>(const bf16*, const bf16*, const int32_t*,
                                            const int32_t*, const int32_t*, int, bf16*, bf16*,
                                            int, int, int, int, int, hipStream_t);
template hipError_t reshape_and_cache<float>(const float*, const float*, const int32_t*,
                                             const int32_t*, const int32_t*, int, float*, float*,
                                             int, int, int, int, int, hipStream_t);

}  // namespace dl
