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
//     results);
//   * the whole query group (Hq/Hkv heads sharing the kv head) is handled by
//     the workgroup, so each K/V byte serves all of them;
//   * each KV block is streamed into LDS with coalesced 16-byte loads, while
//     the next block's loads are already in flight in registers;
//   * scores: BS tokens x (256/BS) threads per token, each thread covering a
//     D-slice for all group heads, combined with lane shuffles;
//   * online softmax in the log2 domain per head; PV accumulates 4 output
//     columns x all group heads per thread;
//   * each split writes (o, m, l) in fp32; a second kernel combines the
//     splits in fixed order.
#include "dl_internal.hpp"

namespace dl {

constexpr int kDecThreads = 256;
constexpr int kDecMaxBS = 128;

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int max_context_len, int BS) {
  DecodePlan pl{};
  const int nblk = (max_context_len + BS - 1) / BS;
  const int items = B * Hkv;
  // aim for >= 2048 workgroups at the longest context, at most 8 blocks each
  int want = (2048 + items - 1) / items;
  int cb = (nblk + want - 1) / want;
  if (cb > 8) cb = 8;
  if (cb < 2 && nblk >= 16) cb = 2;
  if (cb < 1) cb = 1;
  pl.chunk_blocks = cb;
  pl.max_splits = nblk > 0 ? (nblk + cb - 1) / cb : 1;
  pl.ws_bytes = (size_t)B * Hq * pl.max_splits * (D + 2) * sizeof(float);
  return pl;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(kDecThreads)
attn_decode_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
                   const int32_t* __restrict__ bt, int max_blocks, const int32_t* __restrict__ ctx,
                   int Hq, int Hkv, int BS, float scale_log2, int chunk_blocks, int max_splits,
                   float* __restrict__ ws, int num_blocks) {
  constexpr int NT = kDecThreads, VE = 16 / sizeof(T);
  constexpr int KLS = D + VE;          // padded LDS row
  constexpr int U = D / 4;             // PV units (4 columns each)
  constexpr int TG = NT / U;           // token groups in PV
  constexpr int VPB_MAX = kDecMaxBS * (D / VE);          // 16 B vectors per K block
  constexpr int LD_IT = (VPB_MAX + NT - 1) / NT;          // per thread, per tensor
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* Ks = reinterpret_cast<T*>(smem_raw);
  T* Vs = Ks + kDecMaxBS * KLS;
  float* Ps = reinterpret_cast<float*>(Vs + kDecMaxBS * KLS);  // [G][BS]
  float* Qs = Ps + G * kDecMaxBS;                              // [G][D]
  float* st = Qs + G * D;                                      // m[G], l[G], alpha[G]
  float* red = reinterpret_cast<float*>(smem_raw);             // [TG][G][D], aliases Ks/Vs
  static_assert(TG > 1 && TG * G * D * 4 <= 2 * kDecMaxBS * KLS * (int)sizeof(T), "red alias");

  const int b = blockIdx.z, g = blockIdx.y, split = blockIdx.x;
  // lengths beyond the table or the host-declared maximum are clamped, so a
  // violated precondition cannot index outside block_table or the workspace
  const int nblk = min(min((ctx[b] + BS - 1) / BS, max_blocks), max_splits * chunk_blocks);
  const int n = min(ctx[b], nblk * BS);
  const int blk_begin = split * chunk_blocks;
  if (blk_begin >= nblk) return;
  const int blk_end = min(nblk, blk_begin + chunk_blocks);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < G * D; i += NT)
    Qs[i] = to_f32(q[((int64_t)b * Hq + g * G) * D + i]) * scale_log2;
  if (tid < G) {
    st[tid] = -INFINITY;
    st[G + tid] = 0.f;
  }

  const int vpb = BS * (D / VE);
  u32x4 rk[LD_IT], rv[LD_IT];
  auto gload = [&](int blk) {
    int phys = bt[(int64_t)b * max_blocks + blk];
    phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;  // invalid entry: no fault
    const int64_t base = (((int64_t)phys * Hkv + g) * BS) * D;
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int vi = tid + i * NT;
      if (vi < vpb) {
        rk[i] = ld16(kc + base + (int64_t)vi * VE);
        rv[i] = ld16(vc + base + (int64_t)vi * VE);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) {
      const int vi = tid + i * NT;
      if (vi < vpb) {
        const int tok = vi / (D / VE), c = vi % (D / VE);
        st16(Ks + tok * KLS + c * VE, rk[i]);
        st16(Vs + tok * KLS + c * VE, rv[i]);
      }
    }
  };

  // PV ownership
  const int u = tid % U, tg = tid / U;
  float o[G][4];
#pragma unroll
  for (int i = 0; i < G; ++i) o[i][0] = o[i][1] = o[i][2] = o[i][3] = 0.f;

  // score ownership
  const int tpt = NT / BS;           // threads per token (power of 2)
  const int dpt = D / tpt;           // D-slice per thread (multiple of 4)
  const int stok = tid / tpt, part = tid % tpt;

  gload(blk_begin);
  for (int blk = blk_begin; blk < blk_end; ++blk) {
    __syncthreads();  // previous block fully consumed (and Qs / stats visible)
    sstore();
    if (blk + 1 < blk_end) gload(blk + 1);
    __syncthreads();
    const int ntok = min(BS, n - blk * BS);

    // scores
    {
      float acc[G];
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = 0.f;
      const T* kr = Ks + stok * KLS + part * dpt;
      const float* qr = Qs + part * dpt;
      for (int e = 0; e < dpt; e += 4) {
        float kv[4];
        load4(kr + e, kv);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(qr + i * D + e);
          acc[i] += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
        }
      }
      for (int off = tpt >> 1; off > 0; off >>= 1)
#pragma unroll
        for (int i = 0; i < G; ++i) acc[i] += __shfl_xor(acc[i], off, kWave);
      if (part == 0)
#pragma unroll
        for (int i = 0; i < G; ++i) Ps[i * kDecMaxBS + stok] = stok < ntok ? acc[i] : -INFINITY;
    }
    __syncthreads();

    // online softmax, one wave per head
    for (int i = wave; i < G; i += NT / kWave) {
      float mx = -INFINITY;
      for (int t = lane; t < BS; t += kWave) mx = fmaxf(mx, Ps[i * kDecMaxBS + t]);
      mx = wave_max(mx);
      const float m_old = st[i];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int t = lane; t < BS; t += kWave) {
        const float p = exp2f(Ps[i * kDecMaxBS + t] - m_new);
        Ps[i * kDecMaxBS + t] = p;
        sum += p;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float alpha = exp2f(m_old - m_new);
        st[i] = m_new;
        st[G + i] = st[G + i] * alpha + sum;
        st[2 * G + i] = alpha;
      }
    }
    __syncthreads();

    // PV
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float a = st[2 * G + i];
      o[i][0] *= a;
      o[i][1] *= a;
      o[i][2] *= a;
      o[i][3] *= a;
    }
    for (int t = tg; t < ntok; t += TG) {
      float vv[4];
      load4(Vs + t * KLS + 4 * u, vv);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float p = Ps[i * kDecMaxBS + t];
        o[i][0] += p * vv[0];
        o[i][1] += p * vv[1];
        o[i][2] += p * vv[2];
        o[i][3] += p * vv[3];
      }
    }
  }

  // reduce PV partials over token groups (fixed order), write the split
  __syncthreads();  // Ks / Vs no longer read: reuse them for the reduction
#pragma unroll
  for (int i = 0; i < G; ++i)
    *reinterpret_cast<f32x4*>(red + (tg * G + i) * D + 4 * u) =
        f32x4{o[i][0], o[i][1], o[i][2], o[i][3]};
  __syncthreads();
  const int64_t row0 = ((int64_t)b * Hq + g * G) * max_splits + split;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int i = idx / D, d = idx % D;
    float sacc = 0.f;
    for (int z = 0; z < TG; ++z) sacc += red[(z * G + i) * D + d];
    float* dst = ws + (row0 + (int64_t)i * max_splits) * (D + 2);
    dst[d] = sacc;
    if (d == 0) {
      dst[D] = st[i];
      dst[D + 1] = st[G + i];
    }
  }
}

// Combine the splits of one (sequence, head) in fixed order.
template <typename T, int D>
__global__ void __launch_bounds__(D)
attn_decode_combine(const float* __restrict__ ws, const int32_t* __restrict__ ctx,
                    T* __restrict__ out, int Hq, int BS, int chunk_blocks, int max_splits) {
  const int b = blockIdx.y, h = blockIdx.x, d = threadIdx.x;
  const int nblk = (ctx[b] + BS - 1) / BS;
  const int ns = min((nblk + chunk_blocks - 1) / chunk_blocks, max_splits);
  const float* base = ws + ((int64_t)b * Hq + h) * max_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * (D + 2) + D]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* p = base + s * (D + 2);
    const float w = exp2f(p[D] - M);
    num += w * p[d];
    den += w * p[D + 1];
  }
  out[((int64_t)b * Hq + h) * D + d] = from_f32<T>(num / den);
}

template <typename T, int D, int G>
static hipError_t launch_dec(const T* q, const T* kc, const T* vc, const int32_t* bt,
                             int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int BS,
                             float sl2, const DecodePlan& pl, float* ws, int num_blocks,
                             hipStream_t st) {
  constexpr int KLS = D + 16 / sizeof(T);
  const size_t lds = 2 * (size_t)kDecMaxBS * KLS * sizeof(T) +
                     sizeof(float) * ((size_t)G * kDecMaxBS + (size_t)G * D + 3 * G);
  static bool attr_set = false;  // one attribute call per instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_decode_kernel<T, D, G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(pl.max_splits, Hkv, B);
  hipLaunchKernelGGL((attn_decode_kernel<T, D, G>), grid, dim3(kDecThreads), lds, st, q, kc, vc,
                     bt, max_blocks, ctx, Hq, Hkv, BS, sl2, pl.chunk_blocks, pl.max_splits, ws,
                     num_blocks);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dispatch_g(const T* q, const T* kc, const T* vc, const int32_t* bt,
                             int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int BS,
                             float sl2, const DecodePlan& pl, float* ws, int num_blocks,
                             hipStream_t st) {
  switch (Hq / Hkv) {
    case 1: return launch_dec<T, D, 1>(q, kc, vc, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 2: return launch_dec<T, D, 2>(q, kc, vc, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 4: return launch_dec<T, D, 4>(q, kc, vc, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
    case 8: return launch_dec<T, D, 8>(q, kc, vc, bt, max_blocks, ctx, B, Hq, Hkv, BS, sl2, pl, ws, num_blocks, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t attn_decode_paged(const T* q, const T* k_cache, const T* v_cache,
                             const int32_t* block_table, int max_blocks,
                             const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                             float scale, T* out, const DecodePlan& pl, void* ws, int num_blocks,
                             hipStream_t st) {
  if (B == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  float* w = reinterpret_cast<float*>(ws);
  hipError_t e;
  if (D == 128)
    e = dispatch_g<T, 128>(q, k_cache, v_cache, block_table, max_blocks, context_lens, B, Hq, Hkv,
                           BS, sl2, pl, w, num_blocks, st);
  else if (D == 64)
    e = dispatch_g<T, 64>(q, k_cache, v_cache, block_table, max_blocks, context_lens, B, Hq, Hkv,
                          BS, sl2, pl, w, num_blocks, st);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  if (D == 128)
    hipLaunchKernelGGL((attn_decode_combine<T, 128>), dim3(Hq, B), dim3(128), 0, st, w,
                       context_lens, out, Hq, BS, pl.chunk_blocks, pl.max_splits);
  else
    hipLaunchKernelGGL((attn_decode_combine<T, 64>), dim3(Hq, B), dim3(64), 0, st, w,
                       context_lens, out, Hq, BS, pl.chunk_blocks, pl.max_splits);
  return hipGetLastError();
}

template hipError_t attn_decode_paged<bf16>(const bf16*, const bf16*, const bf16*, const int32_t*,
                                            int, const int32_t*, int, int, int, int, int, float,
                                            bf16*, const DecodePlan&, void*, int, hipStream_t);
template hipError_t attn_decode_paged<float>(const float*, const float*, const float*,
                                             const int32_t*, int, const int32_t*, int, int, int,
                                             int, int, float, float*, const DecodePlan&, void*,
                                             int, hipStream_t);

}  // namespace dl
