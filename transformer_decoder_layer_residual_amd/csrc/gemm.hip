// gemm.hip -- planning, dispatch and entry points of the projection GEMMs
// (gfx950).  The kernels live in gemm_tiled.hpp (general tiled kernel),
// gemm_prefill.hpp (large prefill tiles) and gemm_decode.hpp (decode weight
// stream); maps, epilogues and the split-K reduction in gemm_epi.hpp.
#include <algorithm>
#include <cmath>

#include "gemm_decode.hpp"
#include "gemm_prefill.hpp"
#include "gemm_tiled.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------
static const int kCfgBM[kCfgCount] = {256, 128, 64, 16, 32, 128, 64, 16};
static const int kCfgBN[kCfgCount] = {256, 128, 128, 128, 32, 256, kSkBN, 16};


GemmPlan plan_gemm(int M, int N, int K, bool is_f32, bool paired) {
  GemmPlan pl{};
  const int bk = is_f32 ? 32 : 64;
  auto fits = [&](int c) { return !paired || (N / 2) % (kCfgBN[c] / 2) == 0; };
  auto tiles_n = [&](int c) { return (N + kCfgBN[c] - 1) / kCfgBN[c]; };
  auto tiles = [&](int c) { return ((M + kCfgBM[c] - 1) / kCfgBM[c]) * tiles_n(c); };
  int cfg;
  if (is_f32) {
    cfg = kCfg32s;
  } else if (M <= 16 && K % 32 == 0 && N % 16 == 0 && N / 16 >= 256 && fits(kCfgRow16)) {
    cfg = kCfgRow16;   // decode, a few sequences: row-block weight stream, no partials
  } else if (M <= 64 && fits(kCfgSkinny)) {
    cfg = kCfgSkinny;  // decode: weight streaming
  } else if (M >= 256 && K % 64 == 0 && fits(kCfg256)) {
    // ping-pong kernel; 256-row tiles when they fill the chip, else 128
    // (a round-count model favoured 128-row tiles for 1.5 rounds of 256-row
    // ones, but measured no faster and with more panel traffic).  Long rows
    // (K >= 8192) take 256-row tiles split over K already from half a round
    // of them: the tile's smaller fragment traffic per product term then
    // outweighs the fp32 partial round trip (7B down projection, 2048 x 4096
    // x 11008, inside the layer step: 0.741 against 0.760-0.780 ms cold; at
    // K = 4096, the O projection, the split tiles were 80 against 62 us).
    cfg = (tiles(kCfg256) >= 256 || (tiles(kCfg256) >= 128 && K >= 8192)) ? kCfg256 : kCfgPP128;
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
  if (cfg == kCfgRow16) {
    pl.splits = 1;
    pl.k_per_split = K;
    pl.ws_bytes = 0;
    return pl;
  }
  if (cfg == kCfgSkinny) {
    // stream-K over (tile, 256-k stage) units: splits = the partial slabs
    // per tile (1: none), k_per_split = the stages of a tile
    const int S = (K + kSkKS - 1) / kSkKS, tn = tiles_n(cfg);
    const int W = (int)std::min<int64_t>(kSkGrid, (int64_t)tn * S);
    pl.k_per_split = S;
    pl.splits = sk_max_contributors(tn, S, W);
    pl.ws_bytes = pl.splits > 1 ? (size_t)pl.splits * (size_t)M * (size_t)tn * kSkBN *
                                      sizeof(float) : 0;
    return pl;
  }
  if (cfg == kCfg256) {
    // a last round at most half full: the columns it would cover go out as
    // 128-row tiles (about 0.6 of a 256-row tile's time, measured), taken up
    // by the CUs the full rounds free
    const int tm = (M + 255) / 256, tn = tiles_n(cfg), tm128 = (M + 127) / 128;
    const int full = nt / 256;
    if (nt % 256 && full >= 1) {
      const int big_tn = (256 * full) / tm;
      const int small = (tn - big_tn) * tm128;
      const double now = std::ceil(nt / 256.0);
      const double mixed = std::ceil(tm * big_tn / 256.0) + 0.6 * std::ceil(small / 256.0);
      if (big_tn >= 1 && big_tn < tn && mixed < now - 0.2) pl.mixed_tn = big_tn;
    }
  }
  if (cfg == kCfg256 || cfg == kCfgPP128) {
    // ping-pong tiles: split K when the tiles cover fewer than ~3/4 of the
    // CUs (a few hundred rows against a narrow N, e.g. 64 sequences x 4
    // verification tokens: 32 tiles for the 7B down projection), into about
    // 256 workgroups of at least eight 64-wide k-tiles each
    const int ktl = K / 64;
    int sp = 1, kpt = ktl;
    if (nt < 192 && pl.mixed_tn == 0) {
      sp = std::min((256 + nt - 1) / nt, std::min(ktl / 8, 16));
      if (sp >= 2) {
        kpt = (ktl + sp - 1) / sp;
        sp = (ktl + kpt - 1) / kpt;
      } else {
        sp = 1;
        kpt = ktl;
      }
    }
    pl.splits = sp;
    pl.k_per_split = kpt * 64;
    pl.ws_bytes = sp > 1 ? (size_t)sp * (size_t)M * (size_t)tiles_n(cfg) * 256 * sizeof(float) : 0;
    return pl;
  }
  int splits = 1;
  if (M <= 256) {
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
  const int parts = splitk_parts(pl.splits), per_block = kReduceThreads / parts;
  const int blocks = (int)((work + per_block - 1) / per_block);
  hipLaunchKernelGGL((splitk_reduce<Epi>), dim3(blocks), dim3(kReduceThreads), 0, st, partial,
                     pl.splits, parts, M, NP, C::BN, epi);
  return hipGetLastError();
}

template <class Map, class Epi>
static hipError_t launch_big(const bf16* x, int M, int K, const Map& map, const Epi& epi, int NL,
                             hipStream_t st, int bm = 256, int bk = 64, int mixed_tn = 0,
                             int splits = 1, int kps = 0, void* ws = nullptr) {
  const int tiles_n = (NL + 255) / 256;
  if (splits > 1) {  // K % 64 == 0 (the planner splits only then)
    const int tiles_m = (M + bm - 1) / bm, NP = tiles_n * 256, kpt = kps / 64;
    float* partial = reinterpret_cast<float*>(ws);
    const dim3 grid(tiles_m * tiles_n, splits);
    if (bm == 128)
      hipLaunchKernelGGL((gemm_pp_splitk_kernel<128, 64, Map>), grid, dim3(512), 0, st, x, M, K,
                         map, partial, NP, tiles_m, tiles_n, kpt);
    else
      hipLaunchKernelGGL((gemm_pp_splitk_kernel<256, 64, Map>), grid, dim3(512), 0, st, x, M, K,
                         map, partial, NP, tiles_m, tiles_n, kpt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t work = (int64_t)M * tiles_n * (256 / 8);
    const int parts = splitk_parts(splits), per_block = kReduceThreads / parts;
    hipLaunchKernelGGL((splitk_reduce<Epi>), dim3((int)((work + per_block - 1) / per_block)),
                       dim3(kReduceThreads), 0, st, partial, splits, parts, M, NP, 256, epi);
    return hipGetLastError();
  }
  if (K % 64 == 0 && bm == 256 && mixed_tn > 0 && mixed_tn < tiles_n) {
    const int grid = ((M + 255) / 256) * mixed_tn + ((M + 127) / 128) * (tiles_n - mixed_tn);
    if (bk == 32)
      hipLaunchKernelGGL((gemm_pp_mixed_kernel<32, Map, Epi>), dim3(grid), dim3(512), 0, st, x, M,
                         K, map, epi, mixed_tn, tiles_n);
    else
      hipLaunchKernelGGL((gemm_pp_mixed_kernel<64, Map, Epi>), dim3(grid), dim3(512), 0, st, x, M,
                         K, map, epi, mixed_tn, tiles_n);
    return hipGetLastError();
  }
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

template <class Map, class Epi>
static hipError_t launch_skinny(const bf16* x, int M, int K, const Map& map, const Epi& epi,
                                int NL, const GemmPlan& pl, void* ws, hipStream_t st) {
  const int S = pl.k_per_split;
  const int tiles_n = (NL + kSkBN - 1) / kSkBN;
  if (M > 64 || S != (K + kSkKS - 1) / kSkKS) return hipErrorInvalidValue;
  const int NP = tiles_n * kSkBN;
  const int W = (int)std::min<int64_t>(kSkGrid, (int64_t)tiles_n * S);
  float* partial = pl.splits > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  const dim3 grid(W);
  if (M <= 16)
    hipLaunchKernelGGL((gemm_skinny_kernel<16, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K, map,
                       epi, tiles_n, S, partial, NP);
  else if (M <= 32)
    hipLaunchKernelGGL((gemm_skinny_kernel<32, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K, map,
                       epi, tiles_n, S, partial, NP);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<64, Map, Epi>), grid, dim3(kSkNT), 0, st, x, M, K, map,
                       epi, tiles_n, S, partial, NP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t work = (int64_t)M * tiles_n * (kSkBN / 8);
  hipLaunchKernelGGL((streamk_reduce<Epi>), dim3((int)((work + 255) / 256)), dim3(256), 0, st,
                     partial, M, NP, tiles_n, S, W, epi);
  return hipGetLastError();
}

// Unroll depth, waves and 16-row blocks per workgroup of the row-block
// stream, measured on the 8B- and 70B-shaped decode projections: long rows
// (K >= 14336, the down projections) stream best as 4 waves 8 groups deep, K =
// 8192 as 8 waves 16 deep, shorter rows as 4 waves 16 deep.  Two blocks per
// workgroup (each activation fragment feeding both) paid only for long rows
// with at least 512 blocks -- the 70B down projection, 86.3 -> 82.2 us with a
// cache flush before each launch, as 4 waves 4 groups deep; on the 8B gate/up
// and every K = 8192 projection they were 2-12% slower.
template <class Map, class Epi>
static hipError_t launch_row16(const bf16* x, int M, int K, const Map& map, const Epi& epi, int NL,
                               hipStream_t st) {
  const int nblk = NL / 16;
  if (K >= 14336 && nblk >= 512)
    hipLaunchKernelGGL((gemm_row16_kernel<4, 4, 2, Map, Epi>), dim3((nblk + 1) / 2), dim3(256), 0,
                       st, x, M, K, map, epi, nblk);
  else if (K >= 14336)
    hipLaunchKernelGGL((gemm_row16_kernel<8, 4, 1, Map, Epi>), dim3(nblk), dim3(256), 0, st, x, M,
                       K, map, epi, nblk);
  else if (K >= 8192)
    hipLaunchKernelGGL((gemm_row16_kernel<16, 8, 1, Map, Epi>), dim3(nblk), dim3(512), 0, st, x,
                       M, K, map, epi, nblk);
  else
    hipLaunchKernelGGL((gemm_row16_kernel<16, 4, 1, Map, Epi>), dim3(nblk), dim3(256), 0, st, x,
                       M, K, map, epi, nblk);
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
      case kCfg256:
        return launch_big(x, M, K, mk_map(256, 128), mk_epi(256, 128), NL, st, 256, 64,
                          pl.mixed_tn, pl.splits, pl.k_per_split, ws);
      case kCfgPP128:
        return launch_big(x, M, K, mk_map(256, 128), mk_epi(256, 128), NL, st, 128, 64, 0,
                          pl.splits, pl.k_per_split, ws);
      case kCfg128: return launch_cfg<T, T128>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg64: return launch_cfg<T, T64>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg16: return launch_cfg<T, T16>(x, M, K, mk_map(128, 64), mk_epi(128, 64), NL, pl, ws, st);
      case kCfg32s: return launch_cfg<T, T32s>(x, M, K, mk_map(32, 16), mk_epi(32, 16), NL, pl, ws, st);
      case kCfgSkinny:
        return launch_skinny(x, M, K, mk_map(kSkBN, kSkP), mk_epi(kSkBN, kSkP), NL, pl, ws, st);
      case kCfgRow16:
        return launch_row16(x, M, K, mk_map(16, 8), mk_epi(16, 8), NL, st);
    }
    return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t gemm_qkv_rope(const T* x, const T* wq, const T* wk, const T* wv, const int32_t* pos,
                         const float* cos_sin, int max_pos, T* q, T* k, T* v, int M, int H,
                         int Hq, int Hkv, int D, const GemmPlan& pl, void* ws, hipStream_t st,
                         const KVSink& kv) {
  const int NL = (Hq + 2 * Hkv) * D;
  CacheSink<T> sink;
  sink.kc = static_cast<T*>(kv.k_cache);
  sink.vc = static_cast<T*>(kv.v_cache);
  sink.seq = kv.seq_of_token;
  sink.bt = kv.block_table;
  sink.max_blocks = kv.max_blocks;
  sink.BS = kv.block_size;
  sink.num_blocks = kv.num_blocks;
  return dispatch<T>(
      x, M, H, NL, pl, ws, st,
      [&](int, int P) { return MapQKV<T>{wq, wk, wv, H, Hq, Hkv, D, P}; },
      [&](int, int P) { return EpiRope<T>{q, k, v, pos, cos_sin, Hq, Hkv, D, P, max_pos, sink}; });
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
                                       const GemmPlan&, void*, hipStream_t, const KVSink&);    \
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
