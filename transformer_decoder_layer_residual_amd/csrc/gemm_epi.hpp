// gemm_epi.hpp -- weight-row maps, fused epilogues and the split-K reduction
// shared by every projection GEMM kernel.
//
// Every projection of the layer is C = X W^T: X [M][K] activations, W [N][K]
// weights in [out_features][in_features] layout (the FFN weight shapes given on
// the ascend-transformer-boost fusion page, section "fusion operator matrix").
// Both operands are K-contiguous, so 16-byte global loads land directly in the
// MFMA operand layout.  The weight tile is the MFMA's first operand and the
// activation tile its second; each lane therefore ends up owning four
// consecutive output columns of one row, which gives vector stores.
//
// Output columns are organised in pairs (see dl_internal.hpp): a BN-wide tile
// holds P = BN/2 pair-columns; column j (j < P) and column j + P are owned by
// the same lane.  That lets the epilogues need no data exchange:
//   * QKV + RoPE: pair = (i, i + D/2) of one head -- the rotary pairs of the
//     merged Q/K/V projection with the rotary embedding applied on its output
//     (ops-transformer Llama2-7B page, "single-layer operator call chain");
//   * gate/up + SiLU*mul: pair = (gate row j, up row j) -- MergedMatMul(GateUp)
//     then SiLU and the gate x up product (same paragraph);
//   * down + residual: y = h + acc in fp32 (residual add fused into the last
//     dense layer, ATB fusion-strategy page, "MLP fusion");
//   * plain: O-projection and the unfused chain (N may end in a partial
//     tile; its missing weight rows read as zero and its stores are dropped).
#pragma once

#include "dl_internal.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// weight-row maps: logical column r of tile tn -> pointer to the weight row
// ---------------------------------------------------------------------------
template <typename T>
struct MapPlain {
  const T* W;
  int K, BN, N;
  __device__ const T* row(int tn, int r) const {
    const int n = tn * BN + r;
    return n < N ? W + (int64_t)n * K : nullptr;  // ragged last tile: zero rows
  }
};

template <typename T>
struct MapSwiglu {
  const T *Wg, *Wu;
  int K, P;
  __device__ const T* row(int tn, int r) const {
    return r < P ? Wg + ((int64_t)tn * P + r) * K : Wu + ((int64_t)tn * P + (r - P)) * K;
  }
};

template <typename T>
struct MapQKV {
  const T *Wq, *Wk, *Wv;
  int K, Hq, Hkv, D, P;
  __device__ const T* row(int tn, int r) const {
    const int half = D / 2;
    const int second = r >= P;
    const int pc = tn * P + (second ? r - P : r);
    const int head = pc / half, c = pc - head * half;
    const int in_head = second * half + c;
    if (head < Hq) return Wq + ((int64_t)head * D + in_head) * K;
    if (head < Hq + Hkv) return Wk + ((int64_t)(head - Hq) * D + in_head) * K;
    return Wv + ((int64_t)(head - Hq - Hkv) * D + in_head) * K;
  }
};

// ---------------------------------------------------------------------------
// epilogues: (row m, tile tn, first-half column j (multiple of 4), 4 values of
// columns j..j+3 and 4 values of their partners j+P..j+P+3).  An epilogue that
// reads memory (RoPE table, residual) splits into prefetch(m, tn, j), which
// issues those loads, and the call with their result, so a GEMM can fetch the
// next output group's operands before it does the current group's math and
// stores; the five-argument call does both back to back.  apply8 is the same
// computation for 8 consecutive columns and their partners (j a multiple of
// 8), used where a GEMM hands out its output rows from LDS in row order, so
// that a row's chunks leave as whole 128-byte lines.
// ---------------------------------------------------------------------------
struct NoPre {};
// Plain store; columns at or beyond N (the ragged last tile) are dropped.
// N is a multiple of 16, so a group of 4 columns is either all in or all out.
template <typename To>
struct EpiPlain {
  To* out;
  int ldo, BN, P;
  using Pre = NoPre;
  __device__ Pre prefetch(int, int, int) const { return {}; }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b, const Pre&) const {
    (*this)(m, tn, j, a, b);
  }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    const int n = tn * BN + j;
    To* p = out + (int64_t)m * ldo + n;
    if (n < ldo) store4(p, a[0], a[1], a[2], a[3]);
    if (n + P < ldo) store4(p + P, b[0], b[1], b[2], b[3]);
  }
  __device__ void apply8(int m, int tn, int j, const float* a, const float* b) const {
    const int n = tn * BN + j;
    To* p = out + (int64_t)m * ldo + n;
    if (n < ldo) store8(p, a);
    if (n + P < ldo) store8(p + P, b);
  }
};

struct EpiResid {
  float* out;
  const float* resid;
  int ldo, BN, P;
  struct Pre {
    f32x4 r0, r1;
  };
  __device__ Pre prefetch(int m, int tn, int j) const {
    const int n = tn * BN + j;
    const int64_t o = (int64_t)m * ldo + n;
    Pre p{};
    if (n < ldo) p.r0 = *reinterpret_cast<const f32x4*>(resid + o);
    if (n + P < ldo) p.r1 = *reinterpret_cast<const f32x4*>(resid + o + P);
    return p;
  }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b, const Pre& p) const {
    const int n = tn * BN + j;
    const int64_t o = (int64_t)m * ldo + n;
    if (n < ldo) store4(out + o, p.r0[0] + a[0], p.r0[1] + a[1], p.r0[2] + a[2], p.r0[3] + a[3]);
    if (n + P < ldo)
      store4(out + o + P, p.r1[0] + b[0], p.r1[1] + b[1], p.r1[2] + b[2], p.r1[3] + b[3]);
  }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    (*this)(m, tn, j, a, b, prefetch(m, tn, j));
  }
  __device__ void apply8(int m, int tn, int j, const float* a, const float* b) const {
    const int n = tn * BN + j;
    const int64_t o = (int64_t)m * ldo + n;
    float r[8];
    if (n < ldo) {
      load4(resid + o, r);
      load4(resid + o + 4, r + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] += a[e];
      store8(out + o, r);
    }
    if (n + P < ldo) {
      load4(resid + o + P, r);
      load4(resid + o + P + 4, r + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] += b[e];
      store8(out + o + P, r);
    }
  }
};

template <typename To>
struct EpiSwiglu {
  To* out;
  int I, P;
  using Pre = NoPre;
  __device__ Pre prefetch(int, int, int) const { return {}; }
  __device__ void operator()(int m, int tn, int j, f32x4 g, f32x4 u, const Pre&) const {
    (*this)(m, tn, j, g, u);
  }
  __device__ void operator()(int m, int tn, int j, f32x4 g, f32x4 u) const {
    To* p = out + (int64_t)m * I + (int64_t)tn * P + j;
    store4(p, silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2], silu(g[3]) * u[3]);
  }
  __device__ void apply8(int m, int tn, int j, const float* g, const float* u) const {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = silu(g[e]) * u[e];
    store8(out + (int64_t)m * I + (int64_t)tn * P + j, r);
  }
};

// Optional destination of the rotated k and of v in the paged KV cache
// ([num_blocks][Hkv][BS][D]): token m of sequence seq[m] (m itself when seq is
// null) at position pos[m] goes to block bt[seq][pos / BS], slot pos % BS --
// the reshape-and-cache write done in the projection's epilogue (the KV update
// the ascend-transformer-boost fusion page, section "KVCache management", folds
// into the attention block).  Ids outside the table or the pool are skipped.
template <typename To>
struct CacheSink {
  To *kc = nullptr, *vc = nullptr;  // kc == nullptr: no cache write
  const int32_t* seq = nullptr;
  const int32_t* bt = nullptr;
  int max_blocks = 0, BS = 0, num_blocks = 0;
  __device__ To* slot(To* cache, int m, int g, int Hkv, int D, int p) const {
    if (p < 0 || p / BS >= max_blocks) return nullptr;
    const int s = seq ? seq[m] : m;
    const int blk = bt[(int64_t)s * max_blocks + p / BS];
    if (blk < 0 || blk >= num_blocks) return nullptr;
    return cache + (((int64_t)blk * Hkv + g) * BS + p % BS) * D;
  }
};

// Rotate-half RoPE on q and k heads; v passes through.  cos_sin is
// [max_pos][D/2][2] fp32 (cos, sin) built from fp64 angles.  k and v may be
// null when they only go to the cache.
template <typename To>
struct EpiRope {
  To *q, *k, *v;
  const int32_t* pos;
  const float* cs;
  int Hq, Hkv, D, P, max_pos;
  CacheSink<To> sink;
  struct Pre {
    f32x4 c0, c1;  // cos c, sin c, cos c+1, sin c+1 | cos c+2, sin c+2, cos c+3, sin c+3
  };
  __device__ Pre prefetch(int m, int tn, int j) const {
    const int half = D / 2;
    const int pc = tn * P + j;
    const int c = pc % half;
    const int p = min(max(pos[m], 0), max_pos - 1);  // out-of-table positions clamp
    const float* cp = cs + ((int64_t)p * half + c) * 2;
    return Pre{*reinterpret_cast<const f32x4*>(cp), *reinterpret_cast<const f32x4*>(cp + 4)};
  }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    (*this)(m, tn, j, a, b, prefetch(m, tn, j));
  }
  // where pair-column j of tile tn of row m goes: the head row in q/k/v (dst,
  // null when k/v go to the cache only), its cache row (cdst or null), the
  // column c within the first half, and whether it is rotated (q, k) or not (v)
  __device__ void route(int m, int tn, int j, int& c, bool& rot, To*& dst, To*& cdst) const {
    const int half = D / 2;
    const int pc = tn * P + j;
    const int head = pc / half;
    c = pc - head * half;
    cdst = nullptr;
    rot = true;
    if (head < Hq) {
      dst = q + ((int64_t)m * Hq + head) * D;
    } else if (head < Hq + Hkv) {
      const int g = head - Hq;
      dst = k ? k + ((int64_t)m * Hkv + g) * D : nullptr;
      if (sink.kc) cdst = sink.slot(sink.kc, m, g, Hkv, D, pos[m]);
    } else {
      const int g = head - Hq - Hkv;
      dst = v ? v + ((int64_t)m * Hkv + g) * D : nullptr;
      if (sink.kc) cdst = sink.slot(sink.vc, m, g, Hkv, D, pos[m]);
      rot = false;
    }
  }
  __device__ void apply8(int m, int tn, int j, const float* a, const float* b) const {
    const int half = D / 2;
    int c;
    bool rot;
    To *dst, *cdst;
    route(m, tn, j, c, rot, dst, cdst);
    float o1[8], o2[8];
    if (rot) {
      const int p = min(max(pos[m], 0), max_pos - 1);  // out-of-table positions clamp
      const float* cp = cs + ((int64_t)p * half + c) * 2;
      float t[16];  // cos c, sin c, cos c+1, sin c+1, ...
#pragma unroll
      for (int u = 0; u < 4; ++u) load4(cp + 4 * u, t + 4 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o1[e] = a[e] * t[2 * e] - b[e] * t[2 * e + 1];
        o2[e] = b[e] * t[2 * e] + a[e] * t[2 * e + 1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o1[e] = a[e];
        o2[e] = b[e];
      }
    }
    if (dst) {
      store8(dst + c, o1);
      store8(dst + half + c, o2);
    }
    if (cdst) {  // the same rounding as the buffer store: identical bits
      store8(cdst + c, o1);
      store8(cdst + half + c, o2);
    }
  }
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b, const Pre& pf) const {
    const int half = D / 2;
    int c;
    bool rot;
    To *dst, *cdst;
    route(m, tn, j, c, rot, dst, cdst);
    if (rot) {
      const f32x4 c0 = pf.c0, c1 = pf.c1;
      float co[4] = {c0[0], c0[2], c1[0], c1[2]};
      float si[4] = {c0[1], c0[3], c1[1], c1[3]};
      float o1[4], o2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o1[e] = a[e] * co[e] - b[e] * si[e];
        o2[e] = b[e] * co[e] + a[e] * si[e];
      }
      if (dst) {
        store4(dst + c, o1[0], o1[1], o1[2], o1[3]);
        store4(dst + half + c, o2[0], o2[1], o2[2], o2[3]);
      }
      if (cdst) {  // the same rounding as the buffer store: identical bits
        store4(cdst + c, o1[0], o1[1], o1[2], o1[3]);
        store4(cdst + half + c, o2[0], o2[1], o2[2], o2[3]);
      }
    } else {
      if (dst) {
        store4(dst + c, a[0], a[1], a[2], a[3]);
        store4(dst + half + c, b[0], b[1], b[2], b[3]);
      }
      if (cdst) {
        store4(cdst + c, a[0], a[1], a[2], a[3]);
        store4(cdst + half + c, b[0], b[1], b[2], b[3]);
      }
    }
  }
};

// Deterministic split-K reduction followed by the epilogue.  Partials are
// [split][M][NP] with NP = tiles * BN (padded to whole tiles).  A column
// group is (row, tile, 4 first-half columns and their partners).  At decode
// sizes there are few column groups and many splits, so `parts` threads
// share a group: thread p adds splits p, p + parts, ... in order, and the
// parts are added in order through LDS (a fixed order: the result does not
// depend on timing).  One thread per group walking 28 splits took 21 us on a
// 4 x 8192 output.
constexpr int kReduceThreads = 256;

// Threads per column group for a given split count (a power of two <= 8).
inline int splitk_parts(int splits) {
  return splits >= 8 ? 8 : splits >= 4 ? 4 : splits >= 2 ? 2 : 1;
}

template <class Epi>
__global__ void __launch_bounds__(kReduceThreads)
splitk_reduce(const float* __restrict__ partial, int splits, int parts, int M, int NP, int BN,
              Epi epi) {
  __shared__ f32x4 red[kReduceThreads][2];
  const int P = BN / 2, gpt = P / 4, tiles = NP / BN;
  const int per_block = kReduceThreads / parts;
  const int tid = threadIdx.x, cl = tid % per_block, part = tid / per_block;
  const int64_t idx = (int64_t)blockIdx.x * per_block + cl;
  const int64_t total = (int64_t)M * tiles * gpt;
  const bool live = idx < total;
  const int64_t cg = live ? idx : total - 1;
  const int g = (int)(cg % gpt);
  const int64_t rest = cg / gpt;
  const int tn = (int)(rest % tiles);
  const int m = (int)(rest / tiles);
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
  const float* p0 = partial + (int64_t)m * NP + (int64_t)tn * BN + 4 * g;
#pragma unroll 4
  for (int s = part; s < splits; s += parts) {
    const float* p = p0 + (int64_t)s * M * NP;
    a += *reinterpret_cast<const f32x4*>(p);
    b += *reinterpret_cast<const f32x4*>(p + P);
  }
  if (parts > 1) {
    red[tid][0] = a;
    red[tid][1] = b;
    __syncthreads();
    if (part != 0) return;
    for (int q = 1; q < parts; ++q) {
      a += red[cl + q * per_block][0];
      b += red[cl + q * per_block][1];
    }
  }
  if (live) epi(m, tn, 4 * g, a, b);
}

}  // namespace dl
