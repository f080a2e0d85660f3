// gemm.hip -- bf16/fp32 MFMA projection GEMMs with fused epilogues (gfx950).
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
//
// Pipeline: global -> registers -> LDS (double buffered, one barrier per K
// tile), MFMA 16x16x32 bf16 (or 16x16x4 fp32) from LDS, fp32 accumulation.
// Tile order is XCD-aware: consecutive workgroup ids are spread round-robin
// over the 8 XCDs, so the id is remapped to give every XCD a contiguous run of
// tiles, walked M-first in groups so neighbours share weight and activation
// tiles in that XCD's L2.
#include <algorithm>
#include <cmath>
#include <utility>

#include "dl_internal.hpp"

namespace dl {

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int MS = BM / (16 * WM);  // 16-row subtiles per wave
  static constexpr int NS = BN / (16 * WN);  // 16-col subtiles per wave
  static_assert(MS >= 1 && NS >= 2 && NS % 2 == 0, "bad tile");
};

template <typename T>
struct KTile {
  static constexpr int BK = 128 / sizeof(T);            // 128 bytes of K per row
  static constexpr int VE = 16 / sizeof(T);             // elements per 16 B vector
  static constexpr int LS = BK + 16 / sizeof(T);        // padded LDS row (144 B)
};

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
// columns j..j+3 and 4 values of their partners j+P..j+P+3)
// ---------------------------------------------------------------------------
// Plain store; columns at or beyond N (the ragged last tile) are dropped.
// N is a multiple of 16, so a group of 4 columns is either all in or all out.
template <typename To>
struct EpiPlain {
  To* out;
  int ldo, BN, P;
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    const int n = tn * BN + j;
    To* p = out + (int64_t)m * ldo + n;
    if (n < ldo) store4(p, a[0], a[1], a[2], a[3]);
    if (n + P < ldo) store4(p + P, b[0], b[1], b[2], b[3]);
  }
};

struct EpiResid {
  float* out;
  const float* resid;
  int ldo, BN, P;
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    const int n = tn * BN + j;
    const int64_t o = (int64_t)m * ldo + n;
    if (n < ldo) {
      const f32x4 r0 = *reinterpret_cast<const f32x4*>(resid + o);
      store4(out + o, r0[0] + a[0], r0[1] + a[1], r0[2] + a[2], r0[3] + a[3]);
    }
    if (n + P < ldo) {
      const f32x4 r1 = *reinterpret_cast<const f32x4*>(resid + o + P);
      store4(out + o + P, r1[0] + b[0], r1[1] + b[1], r1[2] + b[2], r1[3] + b[3]);
    }
  }
};

template <typename To>
struct EpiSwiglu {
  To* out;
  int I, P;
  __device__ void operator()(int m, int tn, int j, f32x4 g, f32x4 u) const {
    To* p = out + (int64_t)m * I + (int64_t)tn * P + j;
    store4(p, silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2], silu(g[3]) * u[3]);
  }
};

// Rotate-half RoPE on q and k heads; v passes through.  cos_sin is
// [max_pos][D/2][2] fp32 (cos, sin) built from fp64 angles.
template <typename To>
struct EpiRope {
  To *q, *k, *v;
  const int32_t* pos;
  const float* cs;
  int Hq, Hkv, D, P, max_pos;
  __device__ void operator()(int m, int tn, int j, f32x4 a, f32x4 b) const {
    const int half = D / 2;
    const int pc = tn * P + j;
    const int head = pc / half, c = pc - head * half;
    To* dst;
    bool rot = true;
    if (head < Hq) {
      dst = q + ((int64_t)m * Hq + head) * D;
    } else if (head < Hq + Hkv) {
      dst = k + ((int64_t)m * Hkv + (head - Hq)) * D;
    } else {
      dst = v + ((int64_t)m * Hkv + (head - Hq - Hkv)) * D;
      rot = false;
    }
    if (rot) {
      const int p = min(max(pos[m], 0), max_pos - 1);  // out-of-table positions clamp
      const float* cp = cs + ((int64_t)p * half + c) * 2;
      f32x4 c0 = *reinterpret_cast<const f32x4*>(cp);      // cos c, sin c, cos c+1, sin c+1
      f32x4 c1 = *reinterpret_cast<const f32x4*>(cp + 4);  // cos c+2, sin c+2, cos c+3, sin c+3
      float co[4] = {c0[0], c0[2], c1[0], c1[2]};
      float si[4] = {c0[1], c0[3], c1[1], c1[3]};
      float o1[4], o2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o1[e] = a[e] * co[e] - b[e] * si[e];
        o2[e] = b[e] * co[e] + a[e] * si[e];
      }
      store4(dst + c, o1[0], o1[1], o1[2], o1[3]);
      store4(dst + half + c, o2[0], o2[1], o2[2], o2[3]);
    } else {
      store4(dst + c, a[0], a[1], a[2], a[3]);
      store4(dst + half + c, b[0], b[1], b[2], b[3]);
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename T, class C, class Map, class Epi>
__global__ void __launch_bounds__(C::NT)
gemm_kernel(const T* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_m, int tiles_n,
            int kps, float* __restrict__ partial, int NL) {
  constexpr int BM = C::BM, BN = C::BN, NT = C::NT, MS = C::MS, NS = C::NS, WN = C::WN;
  constexpr int BK = KTile<T>::BK, VE = KTile<T>::VE, LS = KTile<T>::LS;
  constexpr int RSTEP = NT / 8;                        // rows covered per load pass
  constexpr int A_IT = (BM + RSTEP - 1) / RSTEP;
  constexpr int W_IT = (BN + RSTEP - 1) / RSTEP;
  constexpr int P = BN / 2;
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LS];

  // ---- tile coordinates (XCD-aware, M-grouped) ----
  int bid = blockIdx.x;
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int gsz = GM * tiles_n;
  const int first_m = (bid / gsz) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int tm = first_m + (bid % gsz) % gm;
  const int tn = (bid % gsz) / gm;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int chunk = t & 7, r0 = t >> 3;

  const int k_begin = blockIdx.y * kps;
  const int k_end = min(K, k_begin + kps);
  const int nkt = (k_end - k_begin + BK - 1) / BK;

  const T* xrow[A_IT];
  bool xok[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int r = r0 + i * RSTEP;
    const int m = tm * BM + r;
    xok[i] = (r < BM) && (m < M);
    xrow[i] = X + (int64_t)(xok[i] ? m : 0) * K + chunk * VE;
  }
  const T* wrow[W_IT];
  bool wok[W_IT];
#pragma unroll
  for (int i = 0; i < W_IT; ++i) {
    const int r = r0 + i * RSTEP;
    const T* base = (r < BN) ? map.row(tn, r) : nullptr;  // nullptr: zero row
    wok[i] = base != nullptr;
    wrow[i] = wok[i] ? base + chunk * VE : X;  // never offset a null row pointer
  }

  u32x4 ra[A_IT], rw[W_IT];
  const u32x4 zero = {0, 0, 0, 0};
  auto gload = [&](int k0) {
    const bool kin = (k0 + chunk * VE) < k_end;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) ra[i] = (xok[i] && kin) ? ld16(xrow[i] + k0) : zero;
#pragma unroll
    for (int i = 0; i < W_IT; ++i) rw[i] = (wok[i] && kin) ? ld16(wrow[i] + k0) : zero;
  };
  auto sstore = [&](int buf) {
    T* As = smem[buf];
    T* Ws = As + BM * LS;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int r = r0 + i * RSTEP;
      if (r < BM) st16(As + r * LS + chunk * VE, ra[i]);
    }
#pragma unroll
    for (int i = 0; i < W_IT; ++i) {
      const int r = r0 + i * RSTEP;
      if (r < BN) st16(Ws + r * LS + chunk * VE, rw[i]);
    }
  };

  f32x4 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = 8 * (lane >> 4);
  if (nkt > 0) {
    gload(k_begin);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nkt; ++it) {
    const int cur = it & 1;
    if (it + 1 < nkt) gload(k_begin + (it + 1) * BK);
    const T* As = smem[cur];
    const T* Ws = As + BM * LS;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      Frag<T> wf[NS], xf[MS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int nsub = (s < NS / 2) ? wn * (NS / 2) + s : BN / 32 + wn * (NS / 2) + (s - NS / 2);
        wf[s].load(Ws + (nsub * 16 + fr) * LS + kk + fk);
      }
#pragma unroll
      for (int i = 0; i < MS; ++i) xf[i].load(As + ((wm * MS + i) * 16 + fr) * LS + kk + fk);
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[i][s] = mfma_k32(wf[s], xf[i], acc[i][s]);
    }
    if (it + 1 < nkt) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int m = tm * BM + (wm * MS + i) * 16 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
      const int j = (wn * (NS / 2) + s) * 16 + 4 * (lane >> 4);
      if (partial) {
        float* p = partial + ((int64_t)blockIdx.y * M + m) * NL + (int64_t)tn * BN + j;
        store4(p, acc[i][s][0], acc[i][s][1], acc[i][s][2], acc[i][s][3]);
        const f32x4 b = acc[i][s + NS / 2];
        store4(p + P, b[0], b[1], b[2], b[3]);
      } else {
        epi(m, tn, j, acc[i][s], acc[i][s + NS / 2]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large prefill tile: 256 x 256 x 64, 8 waves (2 x 4), wave tile 128 x 64 made
// of 32 x 32 blocks on v_mfma_f32_32x32x16_bf16 (the bf16 MFMA shape that
// sustains close to the chip's peak; 16x16x32 issues at well under half of it).
// Loads are branch-free (rows past M or N are clamped to valid memory; their
// results are never stored) and only the last K tile, when K is not a
// multiple of 64, takes the zero-filling path.  MFMA fragments of the next
// 16-wide k step are read from LDS while the current step's MFMAs run.
// ---------------------------------------------------------------------------
template <class Map, class Epi>
__global__ void __launch_bounds__(512, 1)
gemm_big_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_m,
                int tiles_n) {
  constexpr int BM = 256, BN = 256, BK = 64, WN = 4, NT = 512;
  constexpr int MS = BM / (32 * 2), NS = BN / (32 * WN);  // 4 x 2 blocks of 32x32
  constexpr int LS = BK + 8;
  constexpr int RSTEP = NT / 8;
  constexpr int A_IT = BM / RSTEP, W_IT = BN / RSTEP;
  static_assert(NS == 2, "one first-half and one partner block per wave");
  __shared__ __attribute__((aligned(16))) bf16 smem[2][(BM + BN) * LS];

  int bid = blockIdx.x;
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int gsz = GM * tiles_n;
  const int first_m = (bid / gsz) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int tm = first_m + (bid % gsz) % gm;
  const int tn = (bid % gsz) / gm;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int chunk = t & 7, r0 = t >> 3;
  const int fr = lane & 31, fk = 8 * (lane >> 5);

  const bf16* xp[A_IT];
  const bf16* wp[W_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int m = min(tm * BM + r0 + i * RSTEP, M - 1);  // clamped: rows >= M never stored
    xp[i] = X + (int64_t)m * K + chunk * 8;
  }
#pragma unroll
  for (int i = 0; i < W_IT; ++i) {
    const bf16* b = map.row(tn, r0 + i * RSTEP);
    wp[i] = (b ? b : X) + chunk * 8;  // missing rows read valid memory; never stored
  }
  const int nkt = (K + BK - 1) / BK;
  const bool ktail = (K % BK) != 0;
  u32x4 ra[A_IT], rw[W_IT];
  const u32x4 zero = {0, 0, 0, 0};
  auto gload = [&](int k0, bool masked) {
    if (!masked) {
#pragma unroll
      for (int i = 0; i < A_IT; ++i) ra[i] = ld16(xp[i] + k0);
#pragma unroll
      for (int i = 0; i < W_IT; ++i) rw[i] = ld16(wp[i] + k0);
    } else {
      const bool kin = k0 + chunk * 8 < K;
#pragma unroll
      for (int i = 0; i < A_IT; ++i) ra[i] = kin ? ld16(xp[i] + k0) : zero;
#pragma unroll
      for (int i = 0; i < W_IT; ++i) rw[i] = kin ? ld16(wp[i] + k0) : zero;
    }
  };
  auto sstore = [&](int buf) {
    bf16* As = smem[buf];
    bf16* Ws = As + BM * LS;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) st16(As + (r0 + i * RSTEP) * LS + chunk * 8, ra[i]);
#pragma unroll
    for (int i = 0; i < W_IT; ++i) st16(Ws + (r0 + i * RSTEP) * LS + chunk * 8, rw[i]);
  };
  bf16x8 fx[2][MS], fw[2][NS];
  auto lds_frags = [&](int buf, int ks, int set) {
    const bf16* As = smem[buf];
    const bf16* Ws = As + BM * LS;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int nsub = (s == 0) ? wn : BN / 64 + wn;  // 32-col blocks: first half, partner half
      fw[set][s] = *reinterpret_cast<const bf16x8*>(Ws + (nsub * 32 + fr) * LS + ks * 16 + fk);
    }
#pragma unroll
    for (int i = 0; i < MS; ++i)
      fx[set][i] = *reinterpret_cast<const bf16x8*>(As + ((wm * MS + i) * 32 + fr) * LS + ks * 16 + fk);
  };
  f32x16 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][s][e] = 0.f;
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int s = 0; s < NS; ++s) acc[i][s] = mfma_32x32x16(fw[set][s], fx[set][i], acc[i][s]);
  };

  gload(0, nkt == 1 && ktail);
  sstore(0);
  __syncthreads();
  lds_frags(0, 0, 0);
  for (int it = 0; it < nkt; ++it) {
    const int cur = it & 1;
    if (it + 1 < nkt) gload((it + 1) * BK, (it + 2 == nkt) && ktail);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) lds_frags(cur, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
    }
    if (it + 1 < nkt) sstore(cur ^ 1);
    __syncthreads();
    if (it + 1 < nkt) lds_frags(cur ^ 1, 0, 0);
  }
  // epilogue: lane owns column m = ... + (lane & 31) and rows n = 8*i + 4*(lane/32) + j
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int m = tm * BM + (wm * MS + i) * 32 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = wn * 32 + 8 * g + 4 * (lane >> 5);
      const f32x4 a = {acc[i][0][4 * g], acc[i][0][4 * g + 1], acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]};
      const f32x4 b = {acc[i][1][4 * g], acc[i][1][4 * g + 1], acc[i][1][4 * g + 2], acc[i][1][4 * g + 3]};
      epi(m, tn, j, a, b);
    }
  }
}

// ---------------------------------------------------------------------------
// Ping-pong prefill tile: BM x 256 x 64, 8 waves in two groups of 4.
//
// Group g computes output rows [128 g, 128 g + 128) of the tile; each wave a
// 64 x 128 block (2 x 4 blocks of 32 x 32, v_mfma_f32_32x32x16_bf16).  The
// groups run one barrier phase apart: while one group issues its 32 MFMAs for
// k-tile t, the other reads all its MFMA fragments of the next k-tile from
// LDS and issues global->LDS loads, so each SIMD (one wave of each group)
// always has a wave feeding the matrix pipe.
//   group 0: MEM(t) in phase 2t+1, COMP(t) in phase 2t+2
//   group 1: MEM(t) in phase 2t+2, COMP(t) in phase 2t+3
// K-tiles live in two LDS stages; tile t+2 is loaded into tile t's stage in
// phase 2t+3 (after both groups read tile t) and waited for at the end of
// phase 2t+4, before either group reads it.
// Global->LDS loads go straight to LDS (global_load_lds_dwordx4, 1 KB per wave
// instruction = 8 rows of 128 B); the 16-byte chunks of a row are XOR-swizzled
// so the 32-row fragment reads hit distinct banks.  Requires K % 64 == 0.
// ---------------------------------------------------------------------------
// Chunk swizzles (16-byte chunks within an LDS row); both keep the 32-row
// fragment reads conflict-free for 32- and 64-bank LDS models.
template <int BK>
__device__ __forceinline__ int pp_swz(int r) {
  if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);   // 8 chunks per row
  else return ((r >> 1) ^ (r >> 3)) & 3;                      // 4 chunks per row
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BK, class Map, class Epi>
__global__ void __launch_bounds__(512, 1)
gemm_pp_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_m,
               int tiles_n) {
  constexpr int BN = 256;
  constexpr int ROWB = BK * 2;                      // bytes per LDS row
  constexpr int CPR = BK / 8;                       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                     // rows per wave load instruction (1 KB)
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int NSTAGE_FIT = (160 * 1024) / STAGE;
  constexpr int NSTAGE = NSTAGE_FIT < 4 ? NSTAGE_FIT : 4;  // LDS stages (2 .. 4)
  constexpr int LA = NSTAGE - 1;                    // k-tiles loaded ahead
  constexpr int MS = BM / 128, NS = 4;              // 32x32 blocks per wave
  constexpr int KS = BK / 16;                       // k16 steps per tile
  constexpr int RPW = (BM + BN) / 8;                // LDS rows each wave loads per stage
  constexpr int LI = RPW / RPI;                     // load instructions per wave per stage
  constexpr int GR = BM / 2, WR = BM / 4;           // rows per group, per wave
  static_assert(NSTAGE >= 2 && LA <= 3, "stages");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE];

  int bid = blockIdx.x;
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int gsz = GM * tiles_n;
  const int first_m = (bid / gsz) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int tm = first_m + (bid % gsz) % gm;
  const int tn = (bid % gsz) / gm;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int grp = wave >> 2, wig = wave & 3;        // group, wave in group
  const int wm = wig >> 1, wn = wig & 1;
  const int fr = lane & 31, fh = lane >> 5;

  // ---- load assignment: wave w fills LDS rows [RPW w, RPW (w + 1)) of a stage
  // (rows 0..BM-1 = X tile, BM..BM+255 = W tile), RPI rows per instruction.
  const unsigned char* src[LI];
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int row = wave * RPW + i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ pp_swz<BK>(row);   // logical chunk this lane fetches
    const bf16* base;
    if (row < BM) {
      base = X + (int64_t)min(tm * BM + row, M - 1) * K;   // rows >= M: valid, never stored
    } else {
      const bf16* b = map.row(tn, row - BM);
      base = b ? b : X;                                     // missing rows: valid, never stored
    }
    src[i] = reinterpret_cast<const unsigned char*>(base) + c * 16;
  }
  auto issue_loads = [&](int kt) {
    unsigned char* dst = smem + (kt % NSTAGE) * STAGE + wave * RPW * ROWB;
    const int64_t koff = (int64_t)kt * BK * 2;
#pragma unroll
    for (int i = 0; i < LI; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[i] + koff),
          (__attribute__((address_space(3))) void*)(dst + i * RPI * ROWB), 16, 0, 0);
  };
  // wait until k-tile `need` has landed; tiles issued after it may stay in flight
  auto wait_tile = [&](int need, int nkt) {
    const int newer = min(LA - 1, nkt - 1 - need);
    if (newer >= 2) wait_vmcnt<2 * LI>();
    else if (newer == 1) wait_vmcnt<LI>();
    else wait_vmcnt<0>();
  };

  // ---- fragments (all k16 steps of a k-tile)
  bf16x8 fx[KS][MS], fw[KS][NS];
  auto read_frags = [&](int kt) {
    const unsigned char* st = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + fh;                    // logical 16 B chunk
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int r = grp * GR + wm * WR + i * 32 + fr;
        fx[ks][i] = *reinterpret_cast<const bf16x8*>(st + r * ROWB + ((c ^ pp_swz<BK>(r)) << 4));
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int blk = (s < 2) ? 2 * wn + s : 4 + 2 * wn + (s - 2);  // first half, partners
        const int r = BM + blk * 32 + fr;
        fw[ks][s] = *reinterpret_cast<const bf16x8*>(st + r * ROWB + ((c ^ pp_swz<BK>(r)) << 4));
      }
    }
  };
  f32x16 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][s][e] = 0.f;
  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[i][s] = mfma_32x32x16(fw[ks][s], fx[ks][i], acc[i][s]);
  };
#define DL_PHASE_END()                                     \
  do {                                                     \
    __builtin_amdgcn_sched_barrier(0);                     \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
    __builtin_amdgcn_sched_barrier(0);                     \
  } while (0)

  // Phases: group 0 does MEM(t) in phase 2t+1 and COMP(t) in 2t+2; group 1 is
  // one phase later.  Tile t+LA goes into tile t-1's stage in phase 2t+1 (group
  // 0 from its MEM(t), group 1 from its COMP(t-1)); tile t+1 must have landed
  // by the end of phase 2t+2.
  const int nkt = K / BK;
  for (int i = 0; i <= LA && i < nkt; ++i) issue_loads(i);
  wait_tile(0, nkt);
  DL_PHASE_END();                                   // phase 1 begins
  if (grp == 1) DL_PHASE_END();                     // group 1 starts one phase later
  for (int kt = 0; kt < nkt; ++kt) {
    // MEM(kt)
    read_frags(kt);
    if (grp == 0) {
      if (kt >= 1 && kt + LA < nkt) issue_loads(kt + LA);
    } else {
      if (kt + 1 < nkt) wait_tile(kt + 1, nkt);
    }
    DL_PHASE_END();
    // COMP(kt)
    if (grp == 1 && kt + 1 + LA < nkt) issue_loads(kt + 1 + LA);
    compute();
    if (grp == 0 && kt + 1 < nkt) wait_tile(kt + 1, nkt);
    DL_PHASE_END();
  }
  if (grp == 0) DL_PHASE_END();                     // balance group 1's extra barrier
#undef DL_PHASE_END

  // epilogue: lane owns column m and rows n = 8 q + 4 (lane / 32) + j of each block
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int m = tm * BM + grp * GR + wm * WR + i * 32 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = (2 * wn + b) * 32 + 8 * q + 4 * fh;
        const f32x4 lo = {acc[i][b][4 * q], acc[i][b][4 * q + 1], acc[i][b][4 * q + 2], acc[i][b][4 * q + 3]};
        const f32x4 hi = {acc[i][b + 2][4 * q], acc[i][b + 2][4 * q + 1], acc[i][b + 2][4 * q + 2],
                          acc[i][b + 2][4 * q + 3]};
        epi(m, tn, j, lo, hi);
      }
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMM for decode-sized M (at most 64 activation rows).
//
// Here the weights are read exactly once and dominate the bytes (the
// activation block is at most 64 x K), so the kernel is built to keep HBM
// busy rather than to reuse tiles:
//   * work items are (128 weight rows, K slice) pairs: the 64 pair-columns of
//     a tile and their partners, over NST stages of 256 k;
//   * the grid is persistent (one workgroup per CU), each workgroup walks a
//     contiguous run of items as one unbroken stream of stages: the loads for
//     the next item start while the current one finishes, so no workgroup
//     start or drain idles the memory pipe;
//   * each wave streams its 2 x 16 weight rows straight from HBM into
//     registers in the 16x16x32 MFMA operand layout (lane l holds row l % 16
//     at k = 8 * (l / 16) of each 32-wide k group); two stages are in flight,
//     and each k group's registers are reloaded for two stages ahead as soon
//     as its MFMAs are issued;
//   * the activation rows of a stage are loaded into registers one stage
//     ahead and written to a double-buffered LDS tile (2 x MB x 256 bf16, at
//     most 64 KB); chunk c of row m sits at c ^ (m % 16), so a fragment's 16
//     rows hit distinct banks; one barrier per stage;
//   * one workgroup per CU (all 512 registers per lane), so that the weight
//     stream, not occupancy, hides the memory latency;
//   * every load is issued unconditionally (clamped into valid memory; the
//     activation chunks past a slice are written as zeros, which cancels the
//     clamped weights), so the compiler's in-order load counting stays exact;
//   * MFMA 16x16x32 bf16 with the weight block as first operand: lane l ends
//     with four consecutive output columns of activation row l % 16.
// Splits over K write fp32 partials that splitk_reduce sums in fixed order.
// ---------------------------------------------------------------------------
constexpr int kSkBN = 128, kSkP = 64, kSkNT = 256, kSkKS = 256;
constexpr int kSkGrid = 256;  // persistent workgroups: one per CU of the MI355X

template <int MB, int NST, class Map, class Epi>
__global__ void __launch_bounds__(kSkNT, 1)
gemm_skinny_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_n,
                   int n_items, float* __restrict__ partial, int NP) {
  static_assert(NST % 2 == 0 && NST >= 2, "stage pairs");
  constexpr int NI = MB / 16, G = kSkKS / 32, STAGE_B = MB * kSkKS * 2;
  constexpr int XI = MB / 8;  // activation vectors (16 B) per thread per stage
  constexpr int kc = NST * kSkKS;
  __shared__ __attribute__((aligned(1024))) unsigned char xs[2][STAGE_B];

  // contiguous run of items for this workgroup; item = split * tiles_n + tile
  const int i0 = (int)(((int64_t)blockIdx.x * n_items) / gridDim.x);
  const int i1 = (int)(((int64_t)(blockIdx.x + 1) * n_items) / gridDim.x);
  if (i0 >= i1) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kl = 8 * (lane >> 4);  // this lane's k offset inside a 32-wide group
  const int r = wave * 16 + (lane & 15);

  struct Item {
    const bf16 *w0, *w1;  // this lane's weight rows (block 0 and partner)
    int tn, split, k0, klen;
  };
  auto make = [&](int it) {
    Item x;
    x.tn = it % tiles_n;
    x.split = it / tiles_n;
    x.k0 = x.split * kc;
    x.klen = min(K - x.k0, kc);
    x.w0 = map.row(x.tn, r);
    x.w1 = map.row(x.tn, r + kSkP);
    if (!x.w0) x.w0 = X;  // rows past a ragged N: valid memory, results never stored
    if (!x.w1) x.w1 = X;
    return x;
  };

  // ---- activations of stage st of item x: thread t loads 16-byte vectors
  // v = t + 256 u (row v / 32, chunk v % 32: a row's 512 B by 32 consecutive
  // threads) at the start of the stage before and writes them at its end, so
  // waiting for them leaves that stage's weight reloads in flight; chunk c of
  // row m goes to LDS position c ^ (m % 16).  Rows past M read row M-1 (never
  // stored); k past the slice is written as zero.
  u32x4 xr[XI];
  auto load_x = [&](const Item& x, int st) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int v = t + kSkNT * u, m = v >> 5, c = v & 31;
      const int k = min(st * kSkKS + 8 * c, x.klen - 8);
      xr[u] = ld16(X + (int64_t)min(m, M - 1) * K + x.k0 + k);
    }
  };
  auto store_x = [&](const Item& x, int st, int buf) {
    const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int v = t + kSkNT * u, m = v >> 5, c = v & 31;
      st16(&xs[buf][m * 512 + ((c ^ (m & 15)) << 4)],
           st * kSkKS + 8 * c < x.klen ? xr[u] : zero);
    }
  };
  u32x4 wa[2][G], wb[2][G];
  auto load_group = [&](u32x4 (&w)[2][G], const Item& x, int g, int st) {
    const int e = x.k0 + min(st * kSkKS + 32 * g + kl, x.klen - 8);
    w[0][g] = ld16(x.w0 + e);
    w[1][g] = ld16(x.w1 + e);
  };

  f32x4 acc[2][NI];
  auto zero_acc = [&] {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  const int sw = lane & 15;  // chunk swizzle of this lane's fragment rows

  // One stage st of item cur: next activations' first half load, barrier
  // (this stage's activations visible; the other buffer free), MFMAs with
  // the weight reloads for two stages ahead (which may fall in item nxt),
  // the next activations into the other buffer.  Past the last item, loads
  // repeat the current item's last stage (cached) and feed nothing.
  auto stage = [&](u32x4 (&w)[2][G], auto stc, const Item& cur, const Item& nxt, bool last) {
    constexpr int st = decltype(stc)::value;
    const Item& xa = st + 1 < NST ? cur : (last ? cur : nxt);
    const int sx = st + 1 < NST ? st + 1 : (last ? NST - 1 : 0);
    const Item& wi = st + 2 < NST ? cur : (last ? cur : nxt);
    const int swt = st + 2 < NST ? st + 2 : (last ? NST - 1 : st + 2 - NST);
    load_x(xa, sx);
    // bare barrier: __syncthreads() would also drain the weight loads in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* xst = &xs[st & 1][(lane & 15) * 512];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int off = ((4 * g + (lane >> 4)) ^ sw) * 16;
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, w[0][g]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, w[1][g]);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bf16x8 xf = *reinterpret_cast<const bf16x8*>(xst + i * 16 * 512 + off);
        acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xf, acc[0][i], 0, 0, 0);
        acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xf, acc[1][i], 0, 0, 0);
      }
      load_group(w, wi, g, swt);
      // keep the reload here: the scheduler would otherwise sink it to its
      // use two stages later and serialise the stream
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x(xa, sx, (st + 1) & 1);
  };

  Item cur = make(i0);
  Item nxt = make(min(i0 + 1, i1 - 1));
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(wa, cur, g, 0);
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(wb, cur, g, 1);
  load_x(cur, 0);
  store_x(cur, 0, 0);

  const int j = wave * 16 + 4 * (lane >> 4);
  for (int it = i0; it < i1; ++it) {
    const bool last = it + 1 >= i1;
    zero_acc();
    using std::integral_constant;
    stage(wa, integral_constant<int, 0>{}, cur, nxt, last);
    stage(wb, integral_constant<int, 1>{}, cur, nxt, last);
    if constexpr (NST > 2) {
      stage(wa, integral_constant<int, 2>{}, cur, nxt, last);
      stage(wb, integral_constant<int, 3>{}, cur, nxt, last);
    }
    if constexpr (NST > 4) {
      stage(wa, integral_constant<int, 4>{}, cur, nxt, last);
      stage(wb, integral_constant<int, 5>{}, cur, nxt, last);
      stage(wa, integral_constant<int, 6>{}, cur, nxt, last);
      stage(wb, integral_constant<int, 7>{}, cur, nxt, last);
    }
    static_assert(NST == 2 || NST == 4 || NST == 8, "stage sequence above");
    // lane holds C[n = 4 * (lane / 16) + e][m = 16 * i + lane % 16] of each block
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int m = 16 * i + (lane & 15);
      if (m >= M) continue;
      if (partial) {
        float* p = partial + ((int64_t)cur.split * M + m) * NP + (int64_t)cur.tn * kSkBN + j;
        store4(p, acc[0][i][0], acc[0][i][1], acc[0][i][2], acc[0][i][3]);
        store4(p + kSkP, acc[1][i][0], acc[1][i][1], acc[1][i][2], acc[1][i][3]);
      } else {
        epi(m, cur.tn, j, acc[0][i], acc[1][i]);
      }
    }
    cur = nxt;
    nxt = make(min(it + 2, i1 - 1));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // look-ahead loads past the last item
}

// Deterministic split-K reduction (fixed split order) followed by the
// epilogue.  One thread per (row, tile, group of 4 first-half columns).
// Partials are [split][M][NP] with NP = tiles * BN (padded to whole tiles).
template <class Epi>
__global__ void __launch_bounds__(256)
splitk_reduce(const float* __restrict__ partial, int splits, int M, int NP, int BN, Epi epi) {
  const int P = BN / 2, gpt = P / 4, tiles = NP / BN;
  const int NL = NP;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)M * tiles * gpt;
  if (idx >= total) return;
  const int g = (int)(idx % gpt);
  const int64_t rest = idx / gpt;
  const int tn = (int)(rest % tiles);
  const int m = (int)(rest / tiles);
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
  for (int s = 0; s < splits; ++s) {
    const float* p = partial + ((int64_t)s * M + m) * NL + (int64_t)tn * BN + 4 * g;
    a += *reinterpret_cast<const f32x4*>(p);
    b += *reinterpret_cast<const f32x4*>(p + P);
  }
  epi(m, tn, 4 * g, a, b);
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------
static const int kCfgBM[kCfgCount] = {256, 128, 64, 16, 32, 128, 64};
static const int kCfgBN[kCfgCount] = {256, 128, 128, 128, 32, 256, kSkBN};


GemmPlan plan_gemm(int M, int N, int K, bool is_f32, bool paired) {
  GemmPlan pl{};
  const int bk = is_f32 ? 32 : 64;
  auto fits = [&](int c) { return !paired || (N / 2) % (kCfgBN[c] / 2) == 0; };
  auto tiles_n = [&](int c) { return (N + kCfgBN[c] - 1) / kCfgBN[c]; };
  auto tiles = [&](int c) { return ((M + kCfgBM[c] - 1) / kCfgBM[c]) * tiles_n(c); };
  int cfg;
  if (is_f32) {
    cfg = kCfg32s;
  } else if (M <= 64 && fits(kCfgSkinny)) {
    cfg = kCfgSkinny;  // decode: weight streaming
  } else if (M >= 256 && K % 64 == 0 && fits(kCfg256)) {
    // ping-pong kernel; 256-row tiles when they fill the chip, else 128
    cfg = tiles(kCfg256) >= 256 ? kCfg256 : kCfgPP128;
  } else if (M >= 512) {
    cfg = (fits(kCfg256) && tiles(kCfg256) >= 256) ? kCfg256 : (fits(kCfg128) ? kCfg128 : kCfg32s);
  } else if (M > 16) {
    cfg = fits(kCfg64) ? kCfg64 : kCfg32s;
  } else {
    cfg = fits(kCfg16) ? kCfg16 : kCfg32s;
  }
  pl.cfg = cfg;
  pl.BM = kCfgBM[cfg];
  pl.BN = kCfgBN[cfg];
  const int nt = tiles(cfg);
  const int ktiles = (K + bk - 1) / bk;
  if (cfg == kCfgSkinny) {
    // K slice of 2048, 1024 or 512 (whole stage pairs) with the least modelled
    // time: the persistent workgroups take items in rounds; a round streams one
    // item per busy workgroup at min(40 GB/s, 5.6 TB/s / busy workgroups)
    // (measured per-workgroup and whole-chip streaming rates), plus the fp32
    // partial sums written and re-read at 5.6 TB/s
    int best_kc = 8 * kSkKS;
    double best = 1e300;
    for (int kc = 8 * kSkKS; kc >= 2 * kSkKS; kc /= 2) {
      if (kc >= 2 * K && kc > 2 * kSkKS) continue;  // mostly empty stages
      const int s = (K + kc - 1) / kc;
      const int items = s * nt, full = items / kSkGrid, rest = items % kSkGrid;
      const double item_bytes = (double)kSkBN * std::min(kc, K) * 2;
      auto round = [&](int busy) { return item_bytes / std::min(40e9, 5.6e12 / busy); };
      double t = full * round(kSkGrid) + (rest ? round(rest) : 0.0);
      if (s > 1) t += 2.0 * s * M * nt * kSkBN * 4 / 5.6e12;
      if (t < best * 0.98) {
        best = t;
        best_kc = kc;
      }
    }
    pl.splits = (K + best_kc - 1) / best_kc;
    pl.k_per_split = best_kc;
    pl.ws_bytes = pl.splits > 1 ? (size_t)pl.splits * (size_t)M * (size_t)tiles_n(cfg) * kSkBN *
                                      sizeof(float) : 0;
    return pl;
  }
  int splits = 1;
  const bool single_pass = (cfg == kCfg256 || cfg == kCfgPP128);  // no split-K variant
  if (single_pass) {
    splits = 1;
  } else if (M <= 256) {
    // weight-streaming shapes: enough workgroups to keep HBM busy
    const int want = (1024 + nt - 1) / nt;
    splits = want < 1 ? 1 : want;
    const int max_splits = ktiles / 4 > 0 ? ktiles / 4 : 1;
    if (splits > max_splits) splits = max_splits;
  } else if (nt < 128) {
    const int want = (256 + nt - 1) / nt;
    const int max_splits = ktiles / 8 > 0 ? ktiles / 8 : 1;
    splits = want < max_splits ? want : max_splits;
  }
  int kps = ((ktiles + splits - 1) / splits) * bk;
  splits = (K + kps - 1) / kps;
  pl.k_per_split = kps;
  pl.splits = splits;
  pl.ws_bytes = splits > 1 ? (size_t)splits * (size_t)M * (size_t)tiles_n(cfg) * kCfgBN[cfg] * sizeof(float) : 0;
  return pl;
}

template <typename T, class C, class Map, class Epi>
static hipError_t launch_cfg(const T* x, int M, int K, const Map& map, const Epi& epi, int NL,
                             const GemmPlan& pl, void* ws, hipStream_t st) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (NL + C::BN - 1) / C::BN;
  const int NP = tiles_n * C::BN;
  float* partial = pl.splits > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  dim3 grid(tiles_m * tiles_n, pl.splits);
  hipLaunchKernelGGL((gemm_kernel<T, C, Map, Epi>), grid, dim3(C::NT), 0, st, x, M, K, map, epi,
                     tiles_m, tiles_n, pl.k_per_split, partial, NP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t work = (int64_t)M * tiles_n * (C::BN / 8);
  const int blocks = (int)((work + 255) / 256);
  hipLaunchKernelGGL((splitk_reduce<Epi>), dim3(blocks), dim3(256), 0, st, partial, pl.splits, M,
                     NP, C::BN, epi);
  return hipGetLastError();
}

template <class Map, class Epi>
static hipError_t launch_big(const bf16* x, int M, int K, const Map& map, const Epi& epi, int NL,
                             hipStream_t st, int bm = 256, int bk = 64) {
  const int tiles_n = (NL + 255) / 256;
  if (K % 64 == 0 && bm == 128) {
    const int tiles_m = (M + 127) / 128;
    if (bk == 32)
      hipLaunchKernelGGL((gemm_pp_kernel<128, 32, Map, Epi>), dim3(tiles_m * tiles_n), dim3(512), 0,
                         st, x, M, K, map, epi, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_pp_kernel<128, 64, Map, Epi>), dim3(tiles_m * tiles_n), dim3(512), 0,
                         st, x, M, K, map, epi, tiles_m, tiles_n);
    return hipGetLastError();
  }
  const int tiles_m = (M + 255) / 256;
  if (K % 64 == 0) {
    if (bk == 32)
      hipLaunchKernelGGL((gemm_pp_kernel<256, 32, Map, Epi>), dim3(tiles_m * tiles_n), dim3(512), 0,
                         st, x, M, K, map, epi, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_pp_kernel<256, 64, Map, Epi>), dim3(tiles_m * tiles_n), dim3(512), 0,
                         st, x, M, K, map, epi, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_big_kernel<Map, Epi>), dim3(tiles_m * tiles_n), dim3(512), 0, st, x,
                       M, K, map, epi, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <int MB, class Map, class Epi>
static void launch_skinny_mb(const bf16* x, int M, int K, const Map& map, const Epi& epi, int kc,
                             int tiles_n, int n_items, float* partial, int NP, hipStream_t st) {
  const dim3 grid(std::min(n_items, kSkGrid));
  if (kc == 2 * kSkKS)
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, 2, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K,
                       map, epi, tiles_n, n_items, partial, NP);
  else if (kc == 4 * kSkKS)
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, 4, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K,
                       map, epi, tiles_n, n_items, partial, NP);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, 8, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K,
                       map, epi, tiles_n, n_items, partial, NP);
}

template <class Map, class Epi>
static hipError_t launch_skinny(const bf16* x, int M, int K, const Map& map, const Epi& epi,
                                int NL, const GemmPlan& pl, void* ws, hipStream_t st) {
  const int kc = pl.k_per_split;
  if (M > 64 || (kc != 2 * kSkKS && kc != 4 * kSkKS && kc != 8 * kSkKS)) return hipErrorInvalidValue;
  const int tiles_n = (NL + kSkBN - 1) / kSkBN;
  const int NP = tiles_n * kSkBN;
  const int n_items = tiles_n * pl.splits;
  float* partial = pl.splits > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  if (M <= 16) launch_skinny_mb<16>(x, M, K, map, epi, kc, tiles_n, n_items, partial, NP, st);
  else if (M <= 32) launch_skinny_mb<32>(x, M, K, map, epi, kc, tiles_n, n_items, partial, NP, st);
  else launch_skinny_mb<64>(x, M, K, map, epi, kc, tiles_n, n_items, partial, NP, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t work = (int64_t)M * tiles_n * (kSkBN / 8);
  hipLaunchKernelGGL((splitk_reduce<Epi>), dim3((int)((work + 255) / 256)), dim3(256), 0, st,
                     partial, pl.splits, M, NP, kSkBN, epi);
  return hipGetLastError();
}

typedef Tile<128, 128, 2, 2> T128;
typedef Tile<64, 128, 1, 4> T64;
typedef Tile<16, 128, 1, 4> T16;
typedef Tile<32, 32, 2, 1> T32s;

// Map and epilogue objects need BN / P, which depend on the tile; the factory
// lambdas receive (BN, P) and build them.
template <typename T, class MakeMap, class MakeEpi>
static hipError_t dispatch(const T* x, int M, int K, int NL, const GemmPlan& pl, void* ws,
                           hipStream_t st, MakeMap mk_map, MakeEpi mk_epi) {
  if constexpr (sizeof(T) == 4) {
    if (pl.cfg != kCfg32s) return hipErrorInvalidValue;
    return launch_cfg<T, T32s>(x, M, K, mk_map(32, 16), mk_epi(32, 16), NL, pl, ws, st);
  } else {
    switch (pl.cfg) {
      case kCfg256: return launch_big(x, M, K, mk_map(256, 128), mk_epi(256, 128), NL, st, 256);
      case kCfgPP128: return launch_big(x, M, K, mk_map(256, 128), mk_epi(256, 128), NL, st, 128);
      case kCfg128: return launch_cfg<T, T128>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg64: return launch_cfg<T, T64>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg16: return launch_cfg<T, T16>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg32s: return launch_cfg<T, T32s>(x, M, K, mk_map(32, 16), mk_epi(32, 16), NL, pl, ws, st);
      case kCfgSkinny:
        return launch_skinny(x, M, K, mk_map(kSkBN, kSkP), mk_epi(kSkBN, kSkP), NL, pl, ws, st);
    }
    return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t gemm_qkv_rope(const T* x, const T* wq, const T* wk, const T* wv, const int32_t* pos,
                         const float* cos_sin, int max_pos, T* q, T* k, T* v, int M, int H,
                         int Hq, int Hkv, int D, const GemmPlan& pl, void* ws, hipStream_t st) {
  const int NL = (Hq + 2 * Hkv) * D;
  return dispatch<T>(
      x, M, H, NL, pl, ws, st,
      [&](int, int P) { return MapQKV<T>{wq, wk, wv, H, Hq, Hkv, D, P}; },
      [&](int, int P) { return EpiRope<T>{q, k, v, pos, cos_sin, Hq, Hkv, D, P, max_pos}; });
}

template <typename T, typename To>
hipError_t gemm_linear(const T* x, const T* w, To* out, int M, int N, int K, const GemmPlan& pl,
                       void* ws, hipStream_t st) {
  return dispatch<T>(
      x, M, K, N, pl, ws, st, [&](int BN, int) { return MapPlain<T>{w, K, BN, N}; },
      [&](int BN, int P) { return EpiPlain<To>{out, N, BN, P}; });
}

template <typename T>
hipError_t gemm_linear_resid(const T* x, const T* w, const float* resid, float* out, int M, int N,
                             int K, const GemmPlan& pl, void* ws, hipStream_t st) {
  return dispatch<T>(
      x, M, K, N, pl, ws, st, [&](int BN, int) { return MapPlain<T>{w, K, BN, N}; },
      [&](int BN, int P) { return EpiResid{out, resid, N, BN, P}; });
}

template <typename T>
hipError_t gemm_swiglu(const T* x, const T* wg, const T* wu, T* a, int M, int H, int I,
                       const GemmPlan& pl, void* ws, hipStream_t st) {
  return dispatch<T>(
      x, M, H, 2 * I, pl, ws, st, [&](int, int P) { return MapSwiglu<T>{wg, wu, H, P}; },
      [&](int, int P) { return EpiSwiglu<T>{a, I, P}; });
}

#define DL_INST(T)                                                                              \
  template hipError_t gemm_qkv_rope<T>(const T*, const T*, const T*, const T*, const int32_t*, \
                                       const float*, int, T*, T*, T*, int, int, int, int, int, \
                                       const GemmPlan&, void*, hipStream_t);                   \
  template hipError_t gemm_linear<T, T>(const T*, const T*, T*, int, int, int, const GemmPlan&, \
                                        void*, hipStream_t);                                    \
  template hipError_t gemm_linear_resid<T>(const T*, const T*, const float*, float*, int, int,  \
                                           int, const GemmPlan&, void*, hipStream_t);          \
  template hipError_t gemm_swiglu<T>(const T*, const T*, const T*, T*, int, int, int,           \
                                     const GemmPlan&, void*, hipStream_t);

DL_INST(bf16)
DL_INST(float)
template hipError_t gemm_linear<bf16, float>(const bf16*, const bf16*, float*, int, int, int,
                                             const GemmPlan&, void*, hipStream_t);

}  // namespace dl
