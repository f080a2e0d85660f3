// dl_common.hpp -- shared device helpers for the gfx950 decoder-layer kernels.
//
// Storage types: bf16 is clang's native __bf16 (conversion from float is
// round-to-nearest-even), fp32 is float.  All kernels are written for 64-lane
// CDNA4 wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// 16-byte vector load / store helpers (all callers guarantee 16 B alignment).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Element counts per 16-byte vector.
template <typename T>
struct Vec16 {
  static constexpr int n = 16 / sizeof(T);
};

// Unpack a 16-byte vector of T into floats.
__device__ __forceinline__ void unpack16(u32x4 v, float* out, bf16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i];
    out[2 * i] = __uint_as_float(w << 16);
    out[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(u32x4 v, float* out, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}

// Wave-level reductions (64 lanes) through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// MFMA 16x16 fragments.  One "k32 group" contracts 32 k-values:
//   bf16: one v_mfma_f32_16x16x32_bf16, lane l holds 8 consecutive k of row l%16
//         starting at k = 8*(l/16);
//   fp32: eight v_mfma_f32_16x16x4f32; the lane still holds k = 8*(l/16)+c,
//         c = 0..7, one per instruction.  Both operands use the same k order,
//         so the contraction covers all 32 values.
// Output (both): lane l holds C[4*(l/16) + j][l % 16], j = 0..3, where the
// row index runs over the first operand and the column over the second.
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;

template <>
struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) {
    v = *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ void zero() {
    u32x4 z = {0, 0, 0, 0};
    v = __builtin_bit_cast(bf16x8, z);
  }
};

template <>
struct Frag<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4*>(p);
    hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    lo = f32x4{0.f, 0.f, 0.f, 0.f};
    hi = lo;
  }
};

__device__ __forceinline__ f32x4 mfma_k32(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_k32(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  return c;
}

// 32x32x16 bf16 MFMA: lane l holds 8 consecutive k (from k = 8*(l/32)) of row
// l % 32 for both operands; output lane l holds C[8*i + 4*(l/32) + j][l % 32]
// in element 4*i + j (i, j = 0..3), rows over the first operand.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Store 4 consecutive floats as T.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
// Store 8 consecutive floats as T (one 16-byte store for bf16).
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 w = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3],
              (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
  *reinterpret_cast<bf16x8*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)v[0];
  o[1] = (float)v[1];
  o[2] = (float)v[2];
  o[3] = (float)v[3];
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0];
  o[1] = v[1];
  o[2] = v[2];
  o[3] = v[3];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace dl
