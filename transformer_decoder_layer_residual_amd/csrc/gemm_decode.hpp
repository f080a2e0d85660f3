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
//   * a tile is 128 weight rows (the 64 pair-columns and their partners) over
//     the whole K, in stages of 256 k; the (tile, stage) units are numbered
//     tile-major and every workgroup of the persistent grid (one per CU) takes
//     an equal contiguous run of them (stream-K).  A run is one unbroken
//     stream of stages: the loads for the next unit, also across a tile
//     boundary, start while the current one finishes, so no workgroup start
//     or drain idles the memory pipe, and the runs differ by at most one
//     stage (fixed splits of the K range left whole items over: the 7B
//     gate/up took 12 stages on the busiest workgroup against 10.75 on
//     average);
//   * a workgroup's run covers whole tiles (written through the epilogue) and
//     at most two partial ones at its ends, whose fp32 sums go to slab j of
//     the tile (j: the workgroup's rank among the tile's contributors);
//     streamk_reduce adds a tile's slabs in rank order and runs the epilogue,
//     so the result does not depend on timing.  Against fixed K splits this
//     writes 40-65% fewer partial bytes at the 7B shapes (gate/up 13.5
//     against 22.5 MB, QKV 10.5 against 25, down 8.4 against 22.5);
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
//     activation chunks past K are written as zeros, which cancels the
//     clamped weights), so the compiler's in-order load counting stays exact;
//   * MFMA 16x16x32 bf16 with the weight block as first operand: lane l ends
//     with four consecutive output columns of activation row l % 16.
// ---------------------------------------------------------------------------
constexpr int kSkBN = 128, kSkP = 64, kSkNT = 256, kSkKS = 256;
constexpr int kSkGrid = 256;  // persistent workgroups: one per CU of the MI355X

// Stream-K partition: workgroup w of W takes units [w U / W, (w + 1) U / W);
// the owner of unit u is the largest such w.
__host__ __device__ __forceinline__ int64_t sk_begin(int w, int64_t U, int W) {
  return (int64_t)w * U / W;
}
__host__ __device__ __forceinline__ int sk_owner(int64_t u, int64_t U, int W) {
  return (int)(((u + 1) * W - 1) / U);
}

template <int MB, class Map, class Epi>
__global__ void __launch_bounds__(kSkNT, 1)
gemm_skinny_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_n,
                   int S, float* __restrict__ partial, int NP) {
  constexpr int NI = MB / 16, G = kSkKS / 32, STAGE_B = MB * kSkKS * 2;
  constexpr int RB = kSkKS * 2, CPX = kSkKS / 8;  // bytes and 16-byte chunks of an LDS row
  constexpr int XI = MB * CPX / kSkNT;            // activation vectors (16 B) per thread per stage
  static_assert(XI * kSkNT == MB * CPX, "activation vectors split evenly over the threads");
  __shared__ __attribute__((aligned(1024))) unsigned char xs[2][STAGE_B];

  const int64_t U = (int64_t)tiles_n * S;         // (tile, stage) units, tile-major
  const int W = gridDim.x;
  const int u0 = (int)sk_begin(blockIdx.x, U, W), u1 = (int)sk_begin(blockIdx.x + 1, U, W);
  if (u0 >= u1) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kl = 8 * (lane >> 4);  // this lane's k offset inside a 32-wide group
  const int r = wave * 16 + (lane & 15);

  struct Unit {
    const bf16 *w0, *w1;  // this lane's weight rows (block 0 and partner)
    int tn, k0, klen;
  };
  auto make = [&](int u) {
    Unit x;
    x.tn = u / S;
    x.k0 = (u - x.tn * S) * kSkKS;
    x.klen = min(K - x.k0, kSkKS);
    x.w0 = map.row(x.tn, r);
    x.w1 = map.row(x.tn, r + kSkP);
    if (!x.w0) x.w0 = X;  // rows past a ragged N: valid memory, results never stored
    if (!x.w1) x.w1 = X;
    return x;
  };

  // ---- activations of unit x: thread t loads 16-byte vectors v = t + 256 u
  // (row v / 32, chunk v % 32: a row's 512 B by 32 consecutive threads) at
  // the start of the unit before and writes them at its end, so waiting for
  // them leaves that unit's weight reloads in flight; chunk c of row m goes to
  // LDS position c ^ (m % 16).  Rows past M read row M-1 (never stored); k
  // past K is written as zero.
  u32x4 xr[XI];
  auto load_x = [&](const Unit& x) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int v = t + kSkNT * u, m = v / CPX, c = v % CPX;
      const int k = min(8 * c, x.klen - 8);
      xr[u] = ld16(X + (int64_t)min(m, M - 1) * K + x.k0 + k);
    }
  };
  auto store_x = [&](const Unit& x, int buf) {
    const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int v = t + kSkNT * u, m = v / CPX, c = v % CPX;
      st16(&xs[buf][m * RB + ((c ^ (m & 15)) << 4)], 8 * c < x.klen ? xr[u] : zero);
    }
  };
  u32x4 w[2][G];
  auto load_group = [&](const Unit& x, int g) {
    const int e = x.k0 + min(32 * g + kl, x.klen - 8);
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
  const int j = wave * 16 + 4 * (lane >> 4);

  Unit cur = make(u0);
  Unit nxt = make(min(u0 + 1, u1 - 1));
#pragma unroll
  for (int g = 0; g < G; ++g) load_group(cur, g);
  load_x(cur);
  store_x(cur, 0);
  zero_acc();
  int seg0 = u0;  // first unit of the tile segment being summed
  for (int u = u0; u < u1; ++u) {
    // one unit: the next unit's activations load, barrier (this unit's
    // activations visible; the other buffer free), MFMAs with the weight
    // reloads for the next unit, the next activations into the other
    // buffer.  Past the last unit, loads repeat it (cached) and feed nothing.
    const int buf = (u - u0) & 1;
    load_x(nxt);
    // bare barrier: __syncthreads() would also drain the weight loads in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* xst = &xs[buf][(lane & 15) * RB];
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
      load_group(nxt, g);
      // keep the reload here: the scheduler would otherwise sink it to its
      // use in the next unit and serialise the stream
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x(nxt, buf ^ 1);
    // end of a tile segment: the whole tile through the epilogue, else this
    // workgroup's partial sums into the tile's slab of its rank
    if (u + 1 == u1 || (u + 1) % S == 0) {
      const bool whole = seg0 % S == 0 && (u + 1) % S == 0;
      const int rank = whole ? 0 : blockIdx.x - sk_owner((int64_t)cur.tn * S, U, W);
      // lane holds C[n = 4 * (lane / 16) + e][m = 16 * i + lane % 16] of each block
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int m = 16 * i + (lane & 15);
        if (m >= M) continue;
        if (whole) {
          epi(m, cur.tn, j, acc[0][i], acc[1][i]);
        } else {
          float* p = partial + ((int64_t)rank * M + m) * NP + (int64_t)cur.tn * kSkBN + j;
          store4(p, acc[0][i][0], acc[0][i][1], acc[0][i][2], acc[0][i][3]);
          store4(p + kSkP, acc[1][i][0], acc[1][i][1], acc[1][i][2], acc[1][i][3]);
        }
      }
      zero_acc();
      seg0 = u + 1;
    }
    cur = nxt;
    nxt = make(min(u + 2, u1 - 1));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // look-ahead loads past the last unit
}

// Sums the stream-K slabs of the tiles that several workgroups shared, in
// rank order, and runs the epilogue on them; a tile one workgroup covered
// whole was written by it.  Thread: one (row, 8 pair-columns) of a tile.
template <class Epi>
__global__ void __launch_bounds__(256)
streamk_reduce(const float* __restrict__ partial, int M, int NP, int tiles_n, int S, int W,
               Epi epi) {
  constexpr int P = kSkBN / 2, GPT = P / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)M * tiles_n * GPT;
  if (idx >= total) return;
  const int g = (int)(idx % GPT);
  const int64_t rest = idx / GPT;
  const int tn = (int)(rest % tiles_n);
  const int m = (int)(rest / tiles_n);
  const int64_t U = (int64_t)tiles_n * S;
  const int lo = sk_owner((int64_t)tn * S, U, W), hi = sk_owner((int64_t)tn * S + S - 1, U, W);
  if (hi == lo) return;
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
  const float* p0 = partial + (int64_t)m * NP + (int64_t)tn * kSkBN + 4 * g;
  for (int s = 0; s <= hi - lo; ++s) {
    const float* p = p0 + (int64_t)s * M * NP;
    a += *reinterpret_cast<const f32x4*>(p);
    b += *reinterpret_cast<const f32x4*>(p + P);
  }
  epi(m, tn, 4 * g, a, b);
}

// Slabs a stream-K launch needs: the most workgroups sharing one tile (1: no
// tile is shared, no partials).
inline int sk_max_contributors(int tiles_n, int S, int W) {
  const int64_t U = (int64_t)tiles_n * S;
  int mx = 1;
  for (int tn = 0; tn < tiles_n; ++tn) {
    const int c = sk_owner((int64_t)tn * S + S - 1, U, W) - sk_owner((int64_t)tn * S, U, W) + 1;
    if (c > mx) mx = c;
  }
  return mx;
}

// ---------------------------------------------------------------------------
// Row-block weight stream for at most 16 activation rows (decode batches of
// a few sequences), with no partial sums in memory.
//
// A 16-row block is 8 pair-columns and their 8 partners (P = 8), so N / 16
// blocks cover the output -- 256 and more for every decode projection of the
// 8B- and 70B-shaped layers.  A workgroup owns R consecutive blocks (nblk in
// all; a missing last block is streamed from valid rows and never stored).
// Its NW waves split K into contiguous ranges; each wave streams its range in
// 32-wide k groups, loading the R 16 x 32 weight blocks and the 16 x 32
// activation block straight into the 16x16x32 MFMA operand layout (lane l:
// row l % 16, k = 8 * (l / 16) .. + 7), U groups ahead in registers, and
// accumulates each block into two alternating accumulators (even and odd k
// groups).  With R = 2 every activation fragment feeds two blocks, which
// halves the activation reads from L2 and doubles the bytes a workgroup
// streams.  The waves' 16 x 16 results are merged through LDS in wave order
// (fixed, so results do not depend on timing); wave b then holds block b:
// lane l < 32 has weight rows 4 (l / 16) .. + 3 for activation row l % 16, and
// lane l + 32 their partners, fetched with one cross-lane swap.  Against the
// 128-row stream this removes the fp32 partial round trip and the separate
// reduction launch (the 8B down projection: 25.9 against 34.0 us with its
// reduction).  Activation rows past M read row M - 1 and are never stored.
// ---------------------------------------------------------------------------
template <int U, int NW, int R, class Map, class Epi>
__global__ void __launch_bounds__(NW * 64)
gemm_row16_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int nblk) {
  static_assert(R >= 1 && R <= NW && U % 2 == 0, "row-block shape");
  __shared__ f32x4 red[R][NW][64];
  const int tn0 = blockIdx.x * R;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, kq = 8 * (lane >> 4);
  const int G = K / 32;                       // 32-wide k groups (K % 32 == 0)
  const int gpw = (G + NW - 1) / NW;          // groups per wave; the last may get fewer
  const int g0 = wave * gpw;
  const int ng = max(0, min(gpw, G - g0));
  const int nfull = ng / U;                   // whole chunks of U groups
  const bf16* wp[R];
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const bf16* wrow = tn0 + b < nblk ? map.row(tn0 + b, r) : nullptr;
    if (!wrow) wrow = X;                      // rows past a ragged N: never stored
    wp[b] = wrow + (int64_t)g0 * 32 + kq;
  }
  const bf16* xp = X + (int64_t)min(r, M - 1) * K + (int64_t)g0 * 32 + kq;
  f32x4 acc[R][2];
#pragma unroll
  for (int b = 0; b < R; ++b) acc[b][0] = acc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 wb[U][R], xb[U];
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int b = 0; b < R; ++b) wb[u][b] = ld16(wp[b] + 32 * u);
      xb[u] = ld16(xp + 32 * u);
    }
    for (int c = 0; c < nfull; ++c) {
      // every load unconditional (the last chunk reloads itself), so the
      // compiler's in-order load counting never drains the stream
      const int cn = min(c + 1, nfull - 1);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, xb[u]);
#pragma unroll
        for (int b = 0; b < R; ++b)
          acc[b][u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, wb[u][b]), x, acc[b][u & 1], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < R; ++b) wb[u][b] = ld16(wp[b] + 32 * (cn * U + u));
        xb[u] = ld16(xp + 32 * (cn * U + u));
      }
    }
  }
  for (int g = nfull * U; g < ng; ++g) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, ld16(xp + 32 * g));
#pragma unroll
    for (int b = 0; b < R; ++b)
      acc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, ld16(wp[b] + 32 * g)), x, acc[b][0], 0, 0, 0);
  }
#pragma unroll
  for (int b = 0; b < R; ++b) red[b][wave][lane] = acc[b][0] + acc[b][1];
  __syncthreads();
  if (wave >= R || tn0 + wave >= nblk) return;
  const int b = wave;
  f32x4 s = red[b][0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[b][w][lane];
  f32x4 pr;
#pragma unroll
  for (int e = 0; e < 4; ++e) pr[e] = __shfl_xor(s[e], 32, 64);
  const int m = lane & 15;
  if (lane < 32 && m < M) epi(m, tn0 + b, 4 * (lane >> 4), s, pr);
}

}  // namespace dl
