// gemm_decode.hpp -- persistent weight-streaming bf16 GEMM for decode-sized M.
#pragma once

#include <utility>

#include "gemm_epi.hpp"

namespace dl {

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
//     at k = 8 * (l / 16) of each 32-wide k group); each k group's registers
//     are reloaded for the next stage as soon as its MFMAs are issued, so one
//     stage (16 loads of 16 B per lane) is in flight.  Two stages in flight
//     (two register sets) streamed 4-11% slower on every 64-row decode
//     projection of the 7B layer: a plain one-workgroup-per-CU stream, too,
//     runs at 5.8-5.9 TB/s with 8 or 16 loads in flight per lane and at about
//     3.8 TB/s with 32;
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
  constexpr int RB = kSkKS * 2, CPX = kSkKS / 8;  // bytes and 16-byte chunks of an LDS row
  constexpr int XI = MB * CPX / kSkNT;            // activation vectors (16 B) per thread per stage
  static_assert(XI * kSkNT == MB * CPX, "activation vectors split evenly over the threads");
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
      const int v = t + kSkNT * u, m = v / CPX, c = v % CPX;
      const int k = min(st * kSkKS + 8 * c, x.klen - 8);
      xr[u] = ld16(X + (int64_t)min(m, M - 1) * K + x.k0 + k);
    }
  };
  auto store_x = [&](const Item& x, int st, int buf) {
    const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int v = t + kSkNT * u, m = v / CPX, c = v % CPX;
      st16(&xs[buf][m * RB + ((c ^ (m & 15)) << 4)],
           st * kSkKS + 8 * c < x.klen ? xr[u] : zero);
    }
  };
  u32x4 w[2][G];
  auto load_group = [&](const Item& x, int g, int st) {
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

  // One stage st of item cur: next activations' load, barrier (this stage's
  // activations visible; the other buffer free), MFMAs with the weight
  // reloads for the next stage (which may fall in item nxt), the next
  // activations into the other buffer.  Past the last item, loads repeat the
  // current item's last stage (cached) and feed nothing.
  auto stage = [&](auto stc, const Item& cur, const Item& nxt, bool last) {
    constexpr int st = decltype(stc)::value;
    const Item& xa = st + 1 < NST ? cur : (last ? cur : nxt);
    const int sx = st + 1 < NST ? st + 1 : (last ? NST - 1 : 0);
    const Item& wi = st + 1 < NST ? cur : (last ? cur : nxt);
    const int swt = st + 1 < NST ? st + 1 : (last ? NST - 1 : 0);
    load_x(xa, sx);
    // bare barrier: __syncthreads() would also drain the weight loads in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* xst = &xs[st & 1][(lane & 15) * RB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int off = ((4 * g + (lane >> 4)) ^ sw) * 16;
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, w[0][g]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, w[1][g]);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bf16x8 xf = *reinterpret_cast<const bf16x8*>(xst + i * 16 * RB + off);
        acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xf, acc[0][i], 0, 0, 0);
        acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xf, acc[1][i], 0, 0, 0);
      }
      load_group(wi, g, swt);
      // keep the reload here: the scheduler would otherwise sink it to its
      // use in the next stage and serialise the stream
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x(xa, sx, (st + 1) & 1);
  };

  Item cur = make(i0);
  Item nxt = make(min(i0 + 1, i1 - 1));
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(cur, g, 0);
  load_x(cur, 0);
  store_x(cur, 0, 0);

  const int j = wave * 16 + 4 * (lane >> 4);
  for (int it = i0; it < i1; ++it) {
    const bool last = it + 1 >= i1;
    zero_acc();
    using std::integral_constant;
    stage(integral_constant<int, 0>{}, cur, nxt, last);
    stage(integral_constant<int, 1>{}, cur, nxt, last);
    if constexpr (NST > 2) {
      stage(integral_constant<int, 2>{}, cur, nxt, last);
      stage(integral_constant<int, 3>{}, cur, nxt, last);
    }
    if constexpr (NST > 4) {
      stage(integral_constant<int, 4>{}, cur, nxt, last);
      stage(integral_constant<int, 5>{}, cur, nxt, last);
      stage(integral_constant<int, 6>{}, cur, nxt, last);
      stage(integral_constant<int, 7>{}, cur, nxt, last);
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

// ---------------------------------------------------------------------------
// Row-block weight stream for at most 16 activation rows (decode batches of
// a few sequences), with no partial sums in memory.
//
// One workgroup owns 16 weight rows: 8 pair-columns and their 8 partners (P =
// 8), so N / 16 workgroups cover the output -- 256 and more for every decode
// projection of the 8B- and 70B-shaped layers.  Its NW waves split K into
// contiguous ranges; each wave streams its range in 32-wide k groups, loading
// the 16 x 32 weight block and the 16 x 32 activation block straight into the
// 16x16x32 MFMA operand layout (lane l: row l % 16, k = 8 * (l / 16) .. + 7),
// U groups ahead in registers, and accumulates into two alternating
// accumulators.  The waves' 16 x 16 results are merged through LDS in wave
// order (fixed, so results do not depend on timing); lane l < 32 of wave 0
// then holds weight rows 4 (l / 16) .. + 3 for activation row l % 16, and lane
// l + 32 holds their partners, fetched with one cross-lane swap.  Against the
// 128-row stream this removes the fp32 partial round trip and the separate
// reduction launch (the 8B down projection: 25.9 against 34.0 us with its
// reduction).  Activation rows past M read row M - 1 and are never stored.
// ---------------------------------------------------------------------------
template <int U, int NW, class Map, class Epi>
__global__ void __launch_bounds__(NW * 64)
gemm_row16_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi) {
  __shared__ f32x4 red[NW][64];
  const int tn = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, kq = 8 * (lane >> 4);
  const bf16* wrow = map.row(tn, r);
  if (!wrow) wrow = X;                        // rows past a ragged N: never stored
  const bf16* xrow = X + (int64_t)min(r, M - 1) * K;
  const int G = K / 32;                       // 32-wide k groups (K % 32 == 0)
  const int gpw = (G + NW - 1) / NW;          // groups per wave; the last may get fewer
  const int g0 = wave * gpw;
  const int ng = max(0, min(gpw, G - g0));
  const int nfull = ng / U;                   // whole chunks of U groups
  const bf16* wp = wrow + (int64_t)g0 * 32 + kq;
  const bf16* xp = xrow + (int64_t)g0 * 32 + kq;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  u32x4 wb[U], xb[U];
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wb[u] = ld16(wp + 32 * u);
      xb[u] = ld16(xp + 32 * u);
    }
    for (int c = 0; c < nfull; ++c) {
      // every load unconditional (the last chunk reloads itself), so the
      // compiler's in-order load counting never drains the stream
      const int cn = min(c + 1, nfull - 1);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, wb[u]);
        const bf16x8 b = __builtin_bit_cast(bf16x8, xb[u]);
        if (u & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc0, 0, 0, 0);
        wb[u] = ld16(wp + 32 * (cn * U + u));
        xb[u] = ld16(xp + 32 * (cn * U + u));
      }
    }
  }
  for (int g = nfull * U; g < ng; ++g) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(wp + 32 * g));
    const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(xp + 32 * g));
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc0, 0, 0, 0);
  }
  red[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave != 0) return;
  f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][lane];
  f32x4 pr;
#pragma unroll
  for (int e = 0; e < 4; ++e) pr[e] = __shfl_xor(s[e], 32, 64);
  const int m = lane & 15;
  if (lane < 32 && m < M) epi(m, tn, 4 * (lane >> 4), s, pr);
}

}  // namespace dl
