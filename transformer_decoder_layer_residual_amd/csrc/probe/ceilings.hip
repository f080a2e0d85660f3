// ceilings.hip -- measurement kernels for the achievable rates of one MI355X
// (libdl_probe.so; used by the profiling tool, never by the layer library).
//
//   dlp_stream_read  reads a buffer once with 16-byte loads (grid-stride,
//                    4, 8 or 16 independent loads per lane per trip, 1-16
//                    workgroups per CU): the HBM read rate a streaming
//                    kernel can reach;
//   dlp_copy         copies a buffer with 16-byte loads and stores;
//   dlp_mfma_loop    issues v_mfma_f32_32x32x16_bf16 (kind 0) or
//                    v_mfma_f32_16x16x32_bf16 (kind 1) on register operands
//                    only, eight independent accumulators per wave and 1-4
//                    waves per SIMD: the matrix-core rate with no memory in
//                    the way.
// Every kernel writes one value per thread to `sink` (so nothing is optimised
// away); all accesses stay inside the buffers the caller passes.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kCUs = 256;              // MI355X compute units

template <int UNR>
__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (UNR - 1) * stride < n; i += UNR * stride) {
    u32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= src[i];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ void __launch_bounds__(kThreads)
copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

template <int KIND, int NT>
__global__ void __launch_bounds__(NT)
mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  float total = 0.f;
  if constexpr (KIND == 0) {
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) total += acc[c][e];
  } else {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) total += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  }
  sink[(size_t)blockIdx.x * NT + threadIdx.x] = total;
}

}  // namespace

extern "C" {

// Bytes of `sink` each call needs (the largest grid any call launches).
size_t dlp_sink_bytes(void) {
  const size_t a = (size_t)kCUs * 16 * kThreads * sizeof(uint32_t);
  const size_t b = (size_t)kCUs * 1024 * sizeof(float);
  return a > b ? a : b;
}

// Flops of one dlp_mfma_loop call with `waves` waves per SIMD.
double dlp_mfma_flops(int kind, int iters, int waves) {
  const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 16 * 16 * 32;
  return per * 8.0 * iters * (4.0 * waves) * kCUs;
}

// 0 on success; 1 for a bad argument (bytes not a multiple of 16, null
// pointers, a shape outside the listed ones); 2 when the launch failed.
// blocks_per_cu 1..16 workgroups of 256 threads per CU; unroll 4, 8 or 16
// independent 16-byte loads per lane per trip.
int dlp_stream_read(const void* src, size_t bytes, void* sink, int blocks_per_cu, int unroll,
                    void* stream) {
  if (!src || !sink || bytes % 16 || blocks_per_cu < 1 || blocks_per_cu > 16) return 1;
  const dim3 grid(kCUs * blocks_per_cu);
  hipStream_t st = (hipStream_t)stream;
  const u32x4* p = (const u32x4*)src;
  if (unroll == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, grid, dim3(kThreads), 0, st, p, bytes / 16, (uint32_t*)sink);
  else if (unroll == 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, grid, dim3(kThreads), 0, st, p, bytes / 16, (uint32_t*)sink);
  else if (unroll == 16)
    hipLaunchKernelGGL(stream_read_kernel<16>, grid, dim3(kThreads), 0, st, p, bytes / 16, (uint32_t*)sink);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int dlp_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(kCUs * 8), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// One workgroup of 256 x waves threads per CU (waves waves per SIMD: 1..3 for
// kind 0, whose eight 16-register accumulators would spill at four, 1..4 for
// kind 1).
int dlp_mfma_loop(int kind, int iters, int waves, void* sink, void* stream) {
  if (!sink || iters < 0 || (kind != 0 && kind != 1) || waves < 1 || waves > (kind == 0 ? 3 : 4))
    return 1;
  hipStream_t st = (hipStream_t)stream;
  float* o = (float*)sink;
#define DLP_MF(K, NT) hipLaunchKernelGGL((mfma_loop_kernel<K, NT>), dim3(kCUs), dim3(NT), 0, st, iters, o)
  if (kind == 0) {
    if (waves == 1) DLP_MF(0, 256);
    else if (waves == 2) DLP_MF(0, 512);
    else DLP_MF(0, 768);
  } else {
    if (waves == 1) DLP_MF(1, 256);
    else if (waves == 2) DLP_MF(1, 512);
    else if (waves == 3) DLP_MF(1, 768);
    else DLP_MF(1, 1024);
  }
#undef DLP_MF
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
