// gemm_prefill.hpp -- large-tile bf16 MFMA GEMMs for prefill-sized M: the
// ping-pong kernel (K % 64 == 0) and the double-buffered 256x256 kernel.
#pragma once

#include <type_traits>

#include "gemm_epi.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// Large prefill tile: 256 x 256 x 64, 8 waves (2 x 4), wave tile 128 x 64 made
// of 32 x 32 blocks on v_mfma_f32_32x32x16_bf16.  It serves only K that is not
// a multiple of 64 (every benchmarked projection takes the ping-pong tile
// below, which runs faster on v_mfma_f32_16x16x32_bf16).
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
// 64 x 128 block (4 x 8 blocks of 16 x 16, v_mfma_f32_16x16x32_bf16; or 2 x 4
// blocks of 32 x 32 with v_mfma_f32_32x32x16_bf16, see kPPMfma16).  The
// groups run one barrier phase apart: while one group issues its MFMAs for
// k-tile t, the other reads all its MFMA fragments of the next k-tile from
// LDS and issues global->LDS loads, so each SIMD (one wave of each group)
// always has a wave feeding the matrix pipe.
//   group 0: MEM(t) in phase 2t+1, COMP(t) in phase 2t+2
//   group 1: MEM(t) in phase 2t+2, COMP(t) in phase 2t+3
// K-tiles live in two to four LDS stages (three weight and two activation
// stages for 256-row tiles); a tile is loaded into the stage of one both groups
// have read, by each group in its own MEM phase (kPPMemPhaseLoads), and waited
// for by the waves that loaded it before the barrier that precedes its first
// read.
// Global->LDS loads go straight to LDS (global_load_lds_dwordx4, 1 KB per wave
// instruction = 8 rows of 128 B); the 16-byte chunks of a row are XOR-swizzled
// so the 16- and 32-row fragment reads hit distinct banks.  Requires K % 64 == 0.
// ---------------------------------------------------------------------------
// Chunk swizzles (16-byte chunks within an LDS row), functions of a row's low
// four bits.  32x32x16 fragments (lane l: row l % 32, chunk c + l / 32): the
// rows of each 8- or 16-lane group fall on distinct banks.  16x16x32
// fragments (lane l: row l % 16, chunk c + l / 16) are also read with lanes l
// and l + 32 -- the same row, chunks c and c + 2 -- in one LDS cycle, so the
// rows that share a bank half (even or odd rows) must take XOR values from
// distinct cosets of {0, 2}, and the 16 rows of a block distinct values
// (with the 32x32 swizzle half of those reads conflicted: LDS bank-conflict
// cycles at half the LDS active cycles).
template <int BK, bool F16>
__device__ __forceinline__ int pp_swz(int r) {
  if constexpr (F16) {
    if constexpr (BK == 64)
      return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2);
    else
      return ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
  } else {
    if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);   // 8 chunks per row
    else return ((r >> 1) ^ (r >> 3)) & 3;                      // 4 chunks per row
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS footprint of one tile shape: the k-tile stages, or the fp32 staging of
// one group's output rows, whichever is larger.  (A third weight stage alone,
// with both groups still issuing their loads in the odd phases, measured no
// faster: 328.6 against 322.9 us for the 7B gate/up product on the 32x32x16
// form of the tile; what pays is moving the issue points, below.)
//
// Loads in MEM phases only (kPPMemPhaseLoads): every group issues its
// global->LDS loads in its own MEM phase, never in front of its MFMAs, and
// the two groups' loads of a k-tile go out in different phases instead of all
// in the odd ones.  Shapes with three or four stages need only a different
// issue point (group 1 loads tile t+LA in MEM(t), whose stage both groups have
// read by then, instead of tile t+1+LA in COMP(t)).  Two-stage shapes (256-row
// tiles, 64-wide k-tiles) split their stages: the activation rows keep two
// and the weight rows get three, which fill the 160 KB exactly; group 0 loads
// the activation rows (tile t+1 in phase 2t+1) and group 1 the weight rows
// (tile t+2 in phase 2t+2).  Measured against issuing in the odd phases: 7B
// gate/up + SiLU.mul 262 against 287 us back to back (276 against 305-309
// with a cache flush before each launch), 8B-GQA down 622 against 693 us.
constexpr bool kPPMemPhaseLoads = true;
// Split stages for 128-row tiles too (two activation stages of 16 KB, four
// weight stages of 32 KB: weight loads three k-tiles ahead instead of two):
// measured slower on the 7B O projection (3-5%) and the QKV's 128-row tiles
// (1.5-2%), the down projection within +-2.5%, so 128-row tiles keep their
// three whole stages.
constexpr bool kPPSplit128 = false;

template <int BM, int BK>
struct PPGeom {
  static constexpr int BN = 256;
  static constexpr int STAGE = (BM + BN) * BK * 2;
  static constexpr int NSTAGE_FIT = (160 * 1024) / STAGE;
  static constexpr int NSTAGE = NSTAGE_FIT < 4 ? NSTAGE_FIT : 4;  // LDS stages (2 .. 4)
  static constexpr bool SPLIT =
      kPPMemPhaseLoads && BK == 64 && (BM == 256 || (BM == 128 && kPPSplit128));
  static constexpr int XST = BM * BK * 2, WST = BN * BK * 2;  // split: activation, weight stage
  static constexpr int NWS_FIT = (160 * 1024 - 2 * XST) / WST;
  static constexpr int NWS = NWS_FIT < 4 ? NWS_FIT : 4;      // split: weight stages (3 or 4)
  static constexpr int OPITCH = BN + 8;             // fp32 row pitch of the output staging
  static constexpr int MAIN = SPLIT ? 2 * XST + NWS * WST : NSTAGE * STAGE;
  static constexpr int OUT = (BM / 2) * OPITCH * 4;
  static constexpr int SMEM = MAIN > OUT ? MAIN : OUT;
  static_assert(SMEM <= 160 * 1024, "LDS");
};

// Matrix instruction of the ping-pong tile: false = v_mfma_f32_32x32x16_bf16
// (32 x 32 output blocks, k16 steps), true = v_mfma_f32_16x16x32_bf16 (16 x 16
// blocks, k32 steps).  Both read the same LDS bytes per product term from the
// same row layout, each with its own chunk swizzle (pp_swz): every fragment
// row of a lane is its lane row plus a multiple of 16, and a swizzle depends
// on a row's low four bits only.
// The 16x16x32 form is the faster one on the MI355X: register-only loops
// sustain 2.14 against 1.92 PFLOP/s, and the 7B prefill projections ran 3-11%
// faster with it (gate/up + SiLU.mul 290-297 against 326-333 us back to back).
constexpr bool kPPMfma16 = true;
// Wave arrangement of 128-row tiles: false = 2 x 2 waves per group (32 rows x
// 128 columns each), true = 1 x 4 (64 x 64: a fifth fewer fragment reads per
// product term; the 7B O and down projections 2-6% faster).
constexpr bool kPP128Rows1 = true;

// One BM x 256 output tile: tile `bid` of a tiles_m x tiles_n grid whose
// N-tiles start at tn0 (so a launch may cover a range of N with one shape);
// k-tiles kt0 .. kt0 + nkt - 1 are summed (the whole K unless split).
template <int BM, int BK, class Map, class Epi>
__device__ __forceinline__ void pp_tile(const bf16* __restrict__ X, int M, int K, const Map& map,
                                        const Epi& epi, int bid, int tiles_m, int tiles_n,
                                        int tn0, unsigned char* smem, int kt0, int nkt) {
  using Geo = PPGeom<BM, BK>;
  constexpr int BN = 256;
  constexpr int ROWB = BK * 2;                      // bytes per LDS row
  constexpr int CPR = BK / 8;                       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                     // rows per wave load instruction (1 KB)
  constexpr int STAGE = Geo::STAGE;
  constexpr int NSTAGE = Geo::NSTAGE;
  constexpr int LA = NSTAGE - 1;                    // k-tiles loaded ahead
  constexpr bool F16 = kPPMfma16;
  constexpr int MB = F16 ? 16 : 32;                 // rows of an MFMA output block
  // waves of a group along rows x columns: 2 x 2, or 1 x 4 for 128-row tiles
  // with kPP128Rows1 (a wave then holds 64 rows x 64 columns)
  constexpr int WGN = (BM == 128 && kPP128Rows1) ? 4 : 2, WGM = 4 / WGN;
  constexpr int GR = BM / 2, WR = GR / WGM;         // rows per group, per wave
  constexpr int MS = WR / MB, NS = 256 / WGN / MB;  // output blocks per wave (rows, columns)
  constexpr int KS = BK / (F16 ? 32 : 16);          // MFMA k steps per tile
  constexpr int RPW = (BM + BN) / 8;                // LDS rows each wave loads per stage
  constexpr int LI = RPW / RPI;                     // load instructions per wave per stage
  static_assert(MS >= 1 && NS >= 2, "wave tile");
  constexpr int OPITCH = Geo::OPITCH;
  static_assert(NSTAGE >= 2 && LA <= 3, "stages");

  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int gsz = GM * tiles_n;
  const int first_m = (bid / gsz) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int tm = first_m + (bid % gsz) % gm;
  const int tn = tn0 + (bid % gsz) / gm;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS bases in SGPRs
  const int grp = wave >> 2, wig = wave & 3;        // group, wave in group
  const int wm = wig / WGN, wn = wig % WGN;
  const int fr = lane & (MB - 1), fh = lane / MB;   // fragment row, k-chunk group

  // ---- load assignment: wave w fills LDS rows [RPW w, RPW (w + 1)) of a stage
  // (rows 0..BM-1 = X tile, BM..BM+255 = W tile), RPI rows per instruction;
  // with split stages group 0's waves fill the X rows (BM / 4 each, LIX
  // instructions) and group 1's the W rows (64 each, LIW instructions).
  constexpr bool SPLIT = Geo::SPLIT;
  constexpr int NWS = Geo::NWS, LAW = NWS - 1;      // split: weight stages, look-ahead
  constexpr int LIX = BM / 4 / RPI, LIW = 64 / RPI;
  constexpr int LIS = SPLIT ? LIW : LI;             // source rows kept per wave
  static_assert(!SPLIT || (LIX <= LIW && LAW >= 2 && LAW <= 3), "split stages");
  const unsigned char* src[LIS];
#pragma unroll
  for (int i = 0; i < LIS; ++i) {
    // (a group-0 wave of a 128-row tile uses only its first LIX entries; the
    // rest point at valid rows and are never loaded)
    const int row = SPLIT ? (grp == 0 ? wave * (BM / 4) + i * RPI + lane / CPR
                                      : BM + (wave - 4) * 64 + i * RPI + lane / CPR)
                          : wave * RPW + i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ pp_swz<BK, F16>(row);  // logical chunk this lane fetches
    const bf16* base;
    if (row < BM) {
      base = X + (int64_t)min(tm * BM + row, M - 1) * K;   // rows >= M: valid, never stored
    } else {
      const bf16* b = map.row(tn, row - BM);
      base = b ? b : X;                                     // missing rows: valid, never stored
    }
    src[i] = reinterpret_cast<const unsigned char*>(base) + (int64_t)kt0 * BK * 2 + c * 16;
  }
  // group 1 issues in its MEM phase (three or four stages; see kPPMemPhaseLoads)
  constexpr bool G1MEM = kPPMemPhaseLoads && LA >= 2;
  auto load_rows = [&](unsigned char* dst, int kt, auto n) {
    const int64_t koff = (int64_t)kt * BK * 2;
#pragma unroll
    for (int i = 0; i < decltype(n)::value; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[i] + koff),
          (__attribute__((address_space(3))) void*)(dst + i * RPI * ROWB), 16, 0, 0);
  };
  auto issue_loads = [&](int kt) {
    if constexpr (SPLIT) {
      if (grp == 0)
        load_rows(smem + (kt % 2) * Geo::XST + wave * (BM / 4) * ROWB, kt,
                  std::integral_constant<int, LIX>());
      else
        load_rows(smem + 2 * Geo::XST + (kt % NWS) * Geo::WST + (wave - 4) * 64 * ROWB, kt,
                  std::integral_constant<int, LIW>());
    } else {
      load_rows(smem + (kt % NSTAGE) * STAGE + wave * RPW * ROWB, kt,
                std::integral_constant<int, LI>());
    }
  };
  // split stages: group 1 waits for weight tile `need` with `newer` later
  // weight tiles of its own still in flight
  auto wait_w = [&](int newer) {
    if (newer >= 2) wait_vmcnt<2 * LIW>();
    else if (newer == 1) wait_vmcnt<LIW>();
    else wait_vmcnt<0>();
  };
  // wait until this wave's part of k-tile `need` has landed; tiles it issued
  // after that one may stay in flight
  auto wait_tile = [&](int need, int nkt) {
    const int newer = min(LA - 1, nkt - 1 - need);
    if (newer >= 2) wait_vmcnt<2 * LI>();
    else if (newer == 1) wait_vmcnt<LI>();
    else wait_vmcnt<0>();
  };

  // ---- fragments (all k steps of a k-tile)
  bf16x8 fx[KS][MS], fw[KS][NS];
  // Every fragment row a lane reads is fr plus a multiple of MB (16 or 32),
  // so its chunk swizzle is pp_swz(fr) for all of them: a lane's offset within
  // a block at k step ks is one of KS values, the rest is wave-uniform.  A k
  // step spans 2 chunks (k16: the two lane halves) or 4 (k32: four lane
  // groups of 16).
  constexpr int CPS = F16 ? 4 : 2;                  // 16-byte chunks per k step
  int lane_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    lane_off[ks] = fr * ROWB + (((ks * CPS + fh) ^ pp_swz<BK, F16>(fr)) << 4);
  auto read_frags = [&](int kt) {
    const unsigned char* xs =
        (SPLIT ? smem + (kt % 2) * Geo::XST : smem + (kt % NSTAGE) * STAGE) + (grp * GR + wm * WR) * ROWB;
    const unsigned char* ws =
        SPLIT ? smem + 2 * Geo::XST + (kt % NWS) * Geo::WST : smem + (kt % NSTAGE) * STAGE + BM * ROWB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // opaque to the optimiser, so the offsets of every fragment are not
      // kept live across the loop as separate registers
      int lo = lane_off[ks];
      asm volatile("" : "+v"(lo));
#pragma unroll
      for (int i = 0; i < MS; ++i)
        fx[ks][i] = *reinterpret_cast<const bf16x8*>(xs + i * MB * ROWB + lo);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // first half (blocks of this wave's 64 columns), then their partners
        const int blk = (s < NS / 2) ? wn * (NS / 2) + s : 128 / MB + wn * (NS / 2) + (s - NS / 2);
        fw[ks][s] = *reinterpret_cast<const bf16x8*>(ws + blk * MB * ROWB + lo);
      }
    }
  };
  using Acc = typename std::conditional<F16, f32x4, f32x16>::type;
  constexpr int AE = F16 ? 4 : 16;                  // accumulator registers per block
  Acc acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < AE; ++e) acc[i][s][e] = 0.f;
  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if constexpr (F16)
            acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[ks][s], fx[ks][i], acc[i][s], 0,
                                                                0, 0);
          else
            acc[i][s] = mfma_32x32x16(fw[ks][s], fx[ks][i], acc[i][s]);
        }
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
  if constexpr (SPLIT) {
    // each wave loads only its own rows (group 0 activations, group 1
    // weights); its wait counts cover its own loads
    if (grp == 0) {
      issue_loads(0);
      if (nkt > 1) issue_loads(1);
      if (nkt > 1) wait_vmcnt<LIX>();
      else wait_vmcnt<0>();
    } else {
#pragma unroll
      for (int j = 0; j < LAW; ++j)
        if (j < nkt) issue_loads(j);
      wait_w(min(LAW - 1, nkt - 1));
    }
    DL_PHASE_END();                                 // phase 1 begins
    if (grp == 1) DL_PHASE_END();                   // group 1 starts one phase later
    for (int kt = 0; kt < nkt; ++kt) {
      // MEM(kt): group 0 loads activation tile kt+1 into tile kt-1's stage
      // (tile 1 came with the prologue); group 1 loads weight tile kt+LAW
      // into tile kt-1's stage and, after its fragment reads, waits for
      // weight tile kt+1, which group 0 reads in the next phase.  Loads go
      // out before the fragment reads (they target another stage): 1-2% less
      // time over the four 7B projections than after them.
      if (grp == 0) {
        if (kt >= 1 && kt + 1 < nkt) issue_loads(kt + 1);
      } else {
        if (kt + LAW < nkt) issue_loads(kt + LAW);
      }
      read_frags(kt);
      if (grp == 1 && kt + 1 < nkt) wait_w(min(LAW - 1, nkt - 2 - kt));
      DL_PHASE_END();
      // COMP(kt); group 0 then waits for activation tile kt+1
      compute();
      if (grp == 0) wait_vmcnt<0>();
      DL_PHASE_END();
    }
  } else {
  for (int i = 0; i <= LA && i < nkt; ++i) issue_loads(i);
  wait_tile(0, nkt);
  DL_PHASE_END();                                   // phase 1 begins
  if (grp == 1) DL_PHASE_END();                     // group 1 starts one phase later
  for (int kt = 0; kt < nkt; ++kt) {
    // MEM(kt)
    if (grp == 0 || G1MEM) {
      if (kt >= 1 && kt + LA < nkt) issue_loads(kt + LA);
    }
    read_frags(kt);
    if (grp == 1) {
      if (kt + 1 < nkt) wait_tile(kt + 1, nkt);
    }
    DL_PHASE_END();
    // COMP(kt)
    if constexpr (!G1MEM) {
      if (grp == 1 && kt + 1 + LA < nkt) issue_loads(kt + 1 + LA);
    }
    compute();
    if (grp == 0 && kt + 1 < nkt) wait_tile(kt + 1, nkt);
    DL_PHASE_END();
  }
  }
  if (grp == 0) DL_PHASE_END();                     // balance group 1's extra barrier
#undef DL_PHASE_END

  // Epilogue through LDS, one group's 128 (BM 256) or 64 (BM 128) rows at a
  // time: the group's waves park their fp32 accumulators row-major in LDS,
  // then all 512 threads take 8-column chunks in row order and run the
  // epilogue on them, so the 16 chunks of an output row (and of its partner
  // half) leave as whole 128-byte lines.  Lane l holds activation row l % 32
  // and weight rows 8 q + 4 (l / 32) + j of each 32x32 block, or activation
  // row l % 16 and weight rows 4 (l / 16) + j of each 16x16 block.
  float* stage = reinterpret_cast<float*>(smem);
  __syncthreads();                                  // every main-loop LDS read is done
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (grp == pass) {
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int r = wm * WR + i * MB + fr;          // row within the group
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int col = (s < NS / 2 ? 0 : BN / 2) + (wn * (NS / 2) + s % (NS / 2)) * MB + 4 * fh;
#pragma unroll
          for (int q = 0; q < AE / 4; ++q)
            *reinterpret_cast<f32x4*>(stage + r * OPITCH + col + 8 * q) =
                f32x4{acc[i][s][4 * q], acc[i][s][4 * q + 1], acc[i][s][4 * q + 2],
                      acc[i][s][4 * q + 3]};
        }
      }
    }
    __syncthreads();
    constexpr int CH = (BN / 2) / 8;                  // 8-column chunks per half row
#pragma unroll
    for (int it = 0; it < GR * CH / 512; ++it) {
      const int idx = t + it * 512;
      const int r = idx / CH, j = (idx % CH) * 8;
      const int m = tm * BM + pass * GR + r;
      if (m < M) {
        float a[8], b[8];
        load4(stage + r * OPITCH + j, a);
        load4(stage + r * OPITCH + j + 4, a + 4);
        load4(stage + r * OPITCH + BN / 2 + j, b);
        load4(stage + r * OPITCH + BN / 2 + j + 4, b + 4);
        epi.apply8(m, tn, j, a, b);
      }
    }
    __syncthreads();
  }
}

template <int BM, int BK, class Map, class Epi>
__global__ void __launch_bounds__(512, 1)
gemm_pp_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int tiles_m,
               int tiles_n) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[PPGeom<BM, BK>::SMEM];
  pp_tile<BM, BK>(X, M, K, map, epi, blockIdx.x, tiles_m, tiles_n, 0, smem, 0, K / BK);
}

// fp32 partial sums of one K split, [M][NP] row-major (NP = tiles_n * 256),
// a tile's first 128 columns and their partners as the epilogues see them.
struct EpiPartial {
  float* out;
  int NP;
  __device__ void apply8(int m, int tn, int j, const float* a, const float* b) const {
    float* p = out + (int64_t)m * NP + tn * 256 + j;
    store8(p, a);
    store8(p + 128, b);
  }
};

// Split-K variant for shapes whose tiles do not fill the chip (a few hundred
// rows against a narrow N): blockIdx.y is the split, which sums kps k-tiles
// into its own partial slab; splitk_reduce adds the slabs in order and runs
// the real epilogue.
template <int BM, int BK, class Map>
__global__ void __launch_bounds__(512, 1)
gemm_pp_splitk_kernel(const bf16* __restrict__ X, int M, int K, Map map,
                      float* __restrict__ partial, int NP, int tiles_m, int tiles_n, int kps) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[PPGeom<BM, BK>::SMEM];
  const int split = blockIdx.y, kt0 = split * kps;
  const int nkt = min(kps, K / BK - kt0);
  EpiPartial epi{partial + (int64_t)split * M * NP, NP};
  pp_tile<BM, BK>(X, M, K, map, epi, blockIdx.x, tiles_m, tiles_n, 0, smem, kt0, nkt);
}

// 256-row tiles for N-tiles [0, big_tn) and 128-row tiles for the rest, in one
// launch: when 256-row tiles would leave a last round at most half full (the
// 7B QKV projection: 384 tiles on 256 CUs), the remaining columns go out as
// twice as many half-height tiles, which the CUs freed by the first round take
// up at once.
template <int BK, class Map, class Epi>
__global__ void __launch_bounds__(512, 1)
gemm_pp_mixed_kernel(const bf16* __restrict__ X, int M, int K, Map map, Epi epi, int big_tn,
                     int tiles_n) {
  constexpr int S256 = PPGeom<256, BK>::SMEM, S128 = PPGeom<128, BK>::SMEM;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S256 > S128 ? S256 : S128];
  const int tm256 = (M + 255) / 256, n_big = tm256 * big_tn;
  if ((int)blockIdx.x < n_big)
    pp_tile<256, BK>(X, M, K, map, epi, blockIdx.x, tm256, big_tn, 0, smem, 0, K / BK);
  else
    pp_tile<128, BK>(X, M, K, map, epi, blockIdx.x - n_big, (M + 127) / 128, tiles_n - big_tn,
                     big_tn, smem, 0, K / BK);
}

}  // namespace dl
