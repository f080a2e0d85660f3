// dl_internal.hpp -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dl_common.hpp"

namespace dl {

// ---------------------------------------------------------------------------
// GEMM planning.  Every projection is C = X W^T with X [M][K] activations and
// W [N][K] weights.  Output columns are processed in "pairs": a tile of BN
// logical columns holds P = BN/2 pair-columns, and column j of the first half
// is paired with column j of the second half (RoPE partners, gate/up partners;
// plain GEMMs just store both halves).  A plan fixes the tile shape and the
// K split; split plans write fp32 partial sums to the workspace and a second
// kernel reduces them and applies the epilogue.
// ---------------------------------------------------------------------------
enum GemmCfg : int {
  kCfg256 = 0,   // BM 256, BN 256, 8 waves: ping-pong kernel (K % 64 == 0) or the
                 // double-buffered big-tile kernel (K tail); bf16 prefill
  kCfg128 = 1,   // BM 128, BN 128, 4 waves (2x2), wave tile 64x64
  kCfg64 = 2,    // BM 64,  BN 128, 4 waves (1x4), wave tile 64x32
  kCfg16 = 3,    // BM 16,  BN 128, 4 waves (1x4), wave tile 16x32
  kCfg32s = 4,   // BM 32,  BN 32,  2 waves (2x1), wave tile 16x32 (small/odd shapes)
  kCfgPP128 = 5, // BM 128, BN 256, 8 waves: ping-pong kernel (K % 64 == 0), bf16
  kCfgSkinny = 6,// M <= 64, BN 128, 4 waves: weight-streaming decode kernel, bf16
  kCfgRow16 = 7, // M <= 16, BN 16: one workgroup per 16 weight rows, K split over
                 // its waves and merged in LDS (no fp32 partials), bf16 decode
  kCfgCount = 8
};

struct GemmPlan {
  int cfg;
  int BM, BN;
  int splits;        // number of K slices (1 = direct epilogue); kCfgSkinny:
                     // most workgroups sharing one column tile (fp32 slabs)
  int k_per_split;   // multiple of the K tile; kCfgSkinny: K stages per tile
  size_t ws_bytes;   // fp32 partials when splits > 1
  int mixed_tn;      // > 0: 256-row tiles for the first mixed_tn N-tiles, 128-row after
};

// N: logical output columns.  paired: the epilogue needs pair partners, so
// P = BN/2 must divide N/2; plain GEMMs accept a ragged last tile (N % 16 == 0).
GemmPlan plan_gemm(int M, int N, int K, bool is_f32, bool paired);

// Where the QKV epilogue also writes k and v: the paged cache through the
// block table (k_cache == nullptr: no cache write).
struct KVSink {
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  const int32_t* seq_of_token = nullptr;  // nullptr: token t belongs to sequence t
  const int32_t* block_table = nullptr;
  int max_blocks = 0, block_size = 0, num_blocks = 0;
};

// Workspace-free variants share kernels; these return hipError_t.  k and v may
// be nullptr when a sink takes them.
template <typename T>
hipError_t gemm_qkv_rope(const T* x, const T* wq, const T* wk, const T* wv, const int32_t* pos,
                         const float* cos_sin, int max_pos, T* q, T* k, T* v, int M, int H,
                         int Hq, int Hkv, int D, const GemmPlan& pl, void* ws, hipStream_t st,
                         const KVSink& kv = KVSink{});
template <typename T, typename To>
hipError_t gemm_linear(const T* x, const T* w, To* out, int M, int N, int K, const GemmPlan& pl,
                       void* ws, hipStream_t st);
template <typename T>
hipError_t gemm_linear_resid(const T* x, const T* w, const float* resid, float* out, int M, int N,
                             int K, const GemmPlan& pl, void* ws, hipStream_t st);
template <typename T>
hipError_t gemm_swiglu(const T* x, const T* wg, const T* wu, T* a, int M, int H, int I,
                       const GemmPlan& pl, void* ws, hipStream_t st);

// ---------------------------------------------------------------------------
// Other kernels
// ---------------------------------------------------------------------------
hipError_t rope_table_fill(float* cos_sin, int max_pos, int D, double theta, hipStream_t st);

template <typename Tin, typename Tout>
hipError_t rmsnorm_residual(const Tin* x, const float* resid_in, float* resid_out, const Tout* gamma,
                            Tout* out, int T, int H, float eps, hipStream_t st);

template <typename T>
hipError_t reshape_and_cache(const T* k, const T* v, const int32_t* seq_of_token,
                             const int32_t* pos, const int32_t* block_table, int max_blocks,
                             T* k_cache, T* v_cache, int T_, int Hkv, int D, int BS,
                             int num_blocks, hipStream_t st);

// INT8 cache: codes [num_blocks][Hkv][BS][D], row scales [num_blocks][Hkv][BS].
template <typename T>
hipError_t reshape_and_cache_q8(const T* k, const T* v, const int32_t* seq_of_token,
                                const int32_t* pos, const int32_t* block_table, int max_blocks,
                                int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                                int T_, int Hkv, int D, int BS, int num_blocks, hipStream_t st);

template <typename T>
hipError_t attn_prefill(const T* q, const T* k, const T* v, const int32_t* cu_seqlens, int B,
                        int max_seqlen, int Hq, int Hkv, int D, float scale, T* out,
                        hipStream_t st);

struct DecodePlan {
  int chunk_blocks;  // KV blocks per split
  int max_splits;    // splits per sequence at max_context_len
  size_t ws_bytes;
  int narrow_ck;     // > 0: layer-dtype caches go through the narrow paged kernel
  int narrow_sp;     //      with splits of narrow_ck keys, narrow_sp of them at most
};
DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int max_context_len, int BS);

template <typename T>
hipError_t attn_decode_paged(const T* q, const T* k_cache, const T* v_cache,
                             const int32_t* block_table, int max_blocks,
                             const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                             float scale, T* out, const DecodePlan& pl, void* ws, int num_blocks,
                             hipStream_t st);
template <typename T>
hipError_t attn_decode_paged_q8(const T* q, const int8_t* k_codes, const int8_t* v_codes,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, int max_blocks,
                                const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                                int BS, float scale, T* out, const DecodePlan& pl, void* ws,
                                int num_blocks, hipStream_t st);

// Keys per split of the narrow paged kernel.
int narrow_split(int B, int Hkv, int max_ctx, int BS);
// Decode step (one token per sequence) through the narrow paged kernel.
template <typename T>
hipError_t attn_decode_narrow(const T* q, const T* k_cache, const T* v_cache,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS,
                              int max_context_len, float scale, T* out, int ck, int max_sp,
                              void* ws, int num_blocks, hipStream_t st);

// Paged attention for q_len >= 1 new tokens per sequence.
struct PagedPlan {
  int narrow;     // 1: at most 32 rows per kv head, the narrow kernel
  int qb;         // query tokens per workgroup tile (128 or 32 rows / group size)
  int max_qt;     // query tiles per sequence at max_q_len
  int ck;         // keys per split
  int max_sp;     // splits per sequence at max_context_len
  size_t ws_bytes;
};
PagedPlan plan_paged(int B, int Hq, int Hkv, int max_q_len, int max_context_len, int BS, int D,
                     int Tq);
template <typename T>
hipError_t attn_paged_qlens(const T* q, const T* k_cache, const T* v_cache,
                            const int32_t* block_table, int max_blocks, const int32_t* cu_q,
                            const int32_t* context_lens, int B, int Tq, int Hq, int Hkv, int D,
                            int BS, int max_context_len, float scale, T* out, const PagedPlan& pl,
                            void* ws, int num_blocks, hipStream_t st);

// Kernel-per-op baseline pieces (the unfused chain).
template <typename T>
hipError_t unf_rope(T* u, const int32_t* pos, const float* cos_sin, int max_pos, int T_, int nh,
                    int D, hipStream_t st);
template <typename T>
hipError_t unf_scores(const T* q, const T* k, const int32_t* cu_seqlens, int B, int S_max,
                      int Hq, int Hkv, int D, float scale, float* S, hipStream_t st);
template <typename T>
hipError_t unf_softmax(const float* S, T* P, const int32_t* lens, bool lens_are_cu, int B,
                       int S_max, int Hq, int rows_per_head, hipStream_t st);
template <typename T>
hipError_t unf_pv(const T* P, const T* v, const int32_t* cu_seqlens, int B, int S_max, int Hq,
                  int Hkv, int D, T* out, hipStream_t st);
template <typename T>
hipError_t unf_dec_attn(const T* q, const T* kc, const T* vc, const int32_t* bt, int max_blocks,
                        const int32_t* ctx, int ctx_max, int B, int Hq, int Hkv, int D, int BS,
                        float scale, float* S, T* P, T* out, int num_blocks, hipStream_t st);
template <typename T>
hipError_t unf_add(const float* a, const T* b, float* out, int64_t n, hipStream_t st);
template <typename T>
hipError_t unf_silu(const T* g, T* out, int64_t n, hipStream_t st);
template <typename T>
hipError_t unf_mul(const T* a, const T* b, T* out, int64_t n, hipStream_t st);

// Validation of the paged-cache index inputs (check.hip): one workgroup,
// writes the OR of the violated DL_CHECK_BIT_* conditions to *word.
hipError_t check_indices(const int32_t* bt, int B, int max_blocks, int num_blocks, int BS,
                         const int32_t* pos, const int32_t* seq, int T, const int32_t* ctx,
                         int max_ctx, const int32_t* cu, int max_seqlen, int32_t* word,
                         hipStream_t st);

}  // namespace dl
