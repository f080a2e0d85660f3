// gemm_tiled.hpp -- general tiled MFMA GEMM (fp32 path, mid-size M, odd
// shapes).
//
// Pipeline: global -> registers -> LDS (double buffered, one barrier per K
// tile), MFMA 16x16x32 bf16 (or 16x16x4 fp32) from LDS, fp32 accumulation.
// Tile order is XCD-aware: consecutive workgroup ids are spread round-robin
// over the 8 XCDs, so the id is remapped to give every XCD a contiguous run of
// tiles, walked M-first in groups so neighbours share weight and activation
// tiles in that XCD's L2.
#pragma once

#include "gemm_epi.hpp"

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

}  // namespace dl
