/*
 * dl_layer.h -- C ABI of the MI355X (gfx950) fused Llama-style decoder layer.
 *
 * The layer is the pre-norm chain named on the ops-transformer Llama2-7B page
 * (seekfood.cn), paragraph "single-layer operator call chain":
 *
 *   x -> RMSNorm -> Q/K/V linear -> rotary embedding -> self-attention (GQA)
 *     -> output linear -> residual add -> RMSNorm -> gate/up linear -> SiLU
 *     -> down linear -> residual add
 *
 * with prefill and decode taking different attention kernels (same page,
 * paragraph "KV cache and operators") and decode reading K/V from a paged
 * cache addressed through block_table and context lengths (ATB KV-cache page,
 * hwcomputing.csdn.net, section "KV cache memory bottleneck").
 *
 * Conventions (every entry point):
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned.  The library never allocates device memory:
 *     scratch space is a caller-provided workspace whose minimum size comes
 *     from the matching *_workspace_size query (the Setup/Execute split of the
 *     ATB operation API, without hidden state).
 *   - `stream` is a hipStream_t (NULL = default stream).  Calls only enqueue
 *     work on it and return; nothing synchronises.
 *   - Weights are [out_features][in_features]; a projection is y = x W^T.
 *   - dtype DL_BF16: weights, gammas, normalised activations, q/k/v, the KV
 *     cache, attention output and FFN intermediate are bf16 (round to nearest
 *     even), every product accumulates in fp32, and the residual stream
 *     (hidden_in, h, hidden_out) is fp32.  DL_F32: everything is fp32.
 *   - KV cache: separate K and V tensors, each [num_blocks][Hkv][BS][D], in
 *     the layer dtype or as INT8 codes with row scales (dl_kv_cache below).
 *     Position p of sequence s lives in physical block
 *     block_table[s][p / BS] at slot p % BS.  block_table is
 *     [B][max_blocks_per_seq] int32; unused entries may hold any value.
 *   - Return value: DL_OK, or an error code, in which case NOTHING was
 *     enqueued; dl_last_error() then describes the failure (thread-local).
 *     DL_ERR_HIP reports a failed launch.
 *   - Device-side preconditions (not checked by the compute calls; a bad
 *     entry gives wrong numbers, never a memory fault, and dl_check_indices
 *     reports it):
 *       block_table entries that are used lie in [0, num_blocks);
 *       0 <= positions[t] < max_blocks_per_seq * BS;
 *       0 <= seq_of_token[t] < number of block_table rows (B);
 *       1 <= context_lens[b] <= max_context_len;
 *       cu_seqlens / cu_q_lens start at 0, never decrease, end at T (Tq), and
 *       no length exceeds max_seqlen (max_q_len).
 *     An out-of-range table entry makes the cache write drop the token and
 *     the attention read block 0 instead; query rows named by a cumulative
 *     length outside [0, T) are not computed.
 *   - Supported shapes: head_dim D in {64, 128}; Hq % Hkv == 0 with
 *     Hq / Hkv in {1, 2, 4, 8}; BS in {16, 32, 64, 128}; hidden H a multiple
 *     of 32 and <= 8192; intermediate I a multiple of 16; reduction sizes a
 *     multiple of 8.  Anything else returns DL_ERR_UNSUPPORTED.
 */
#ifndef DL_LAYER_H
#define DL_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DL_OK = 0,
  DL_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent dims */
  DL_ERR_UNSUPPORTED = 2,  /* shape outside the supported set (see above) */
  DL_ERR_ALIGNMENT = 3,    /* a tensor pointer is not 16-byte aligned */
  DL_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
  DL_ERR_HIP = 5           /* the HIP runtime reported an error */
} dl_status;

typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;

/* DL_FUSED: the fused kernels.  DL_UNFUSED: the kernel-per-op chain (separate
 * q/k/v GEMMs, RoPE pass, score matrix in fp32, softmax, PV, separate gate and
 * up GEMMs, SiLU and multiply passes, residual adds as their own kernels), the
 * "step by step" execution mode of the ascend-transformer-boost page (section
 * "fusion granularity boundaries"), kept as the HBM-bytes baseline. */
typedef enum { DL_FUSED = 0, DL_UNFUSED = 1 } dl_mode;

typedef struct {
  int32_t hidden;        /* H */
  int32_t n_q_heads;     /* Hq */
  int32_t n_kv_heads;    /* Hkv */
  int32_t head_dim;      /* D */
  int32_t intermediate;  /* I */
  int32_t block_size;    /* BS, KV-cache block size in tokens */
  float rms_eps;
  dl_dtype dtype;
} dl_layer_dims;

/* ln1/ln2 gammas [H]; w_q [Hq*D][H]; w_k, w_v [Hkv*D][H]; w_o [H][Hq*D];
 * w_gate, w_up [I][H]; w_down [H][I] (the separate FFN weight shapes of the
 * ascend-transformer-boost page, section "fusion operator matrix"). */
typedef struct {
  const void *ln1_gamma, *w_q, *w_k, *w_v, *w_o, *ln2_gamma, *w_gate, *w_up, *w_down;
} dl_layer_weights;

/*
 * Element format of a KV cache.
 *   DL_KV_LAYER: K and V values in the layer dtype.
 *   DL_KV_INT8:  per-token INT8 quantisation with online scales (ATB KV-cache
 *     page, hwcomputing.csdn.net, section "KV cache quantisation": one fp32
 *     scale for each token's K and one for its V, computed as the token is
 *     written; the paged attention dequantises the blocks as it loads them).
 *     A row is one (token, kv head) D-vector of K or of V; writing it stores
 *       scale = max|x| / 127 and code = x / scale rounded to the nearest
 *       integer (ties to even), clamped to [-127, 127], both in fp32
 *     (an all-zero row stores scale 0 and zero codes); reading it uses
 *     code x scale.  Symmetric: there is no offset.
 */
typedef enum { DL_KV_LAYER = 0, DL_KV_INT8 = 1 } dl_kv_format;

/*
 * A paged KV cache.  A zero-initialised tail (format 0, NULL scales) is the
 * layer-dtype cache.
 *   k_cache, v_cache: [num_blocks][Hkv][BS][D] values (DL_KV_LAYER) or int8
 *     codes (DL_KV_INT8), 16-byte aligned;
 *   k_scale, v_scale: DL_KV_INT8 only, [num_blocks][Hkv][BS] fp32, 4-byte
 *     aligned: the scale of the row at the same (block, head, slot).
 */
typedef struct {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  dl_kv_format format;
  float* k_scale;
  float* v_scale;
} dl_kv_cache;

/* Human-readable name of a status code (static string). */
const char* dl_status_string(dl_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* dl_last_error(void);
/* ABI version of this header (incremented on incompatible change). */
int32_t dl_abi_version(void);

/*
 * RoPE table: cos_sin[p][i][0..1] = cos, sin of p * theta^(-2i/D) for
 * p < max_pos, i < D/2, with the angle computed in fp64 and rounded to fp32.
 * The pages name the rotary embedding on the QKV output without a formula;
 * this is the rotate-half (i, i + D/2) pairing of Llama.
 * cos_sin: device, max_pos * D floats.
 */
dl_status dl_rope_table_fill(float* cos_sin, int32_t max_pos, int32_t head_dim, double theta,
                             void* stream);

/*
 * RMSNorm, optionally fused with the residual add (ascend-transformer-boost
 * page, "fusion operator matrix": norm fused with the residual add; RMSNorm in
 * the Llama chain of the ops-transformer page).
 *   residual_in == NULL: out = gamma * x / sqrt(mean(x^2) + eps)
 *   otherwise:           h = x + residual_in (fp32), written to residual_out
 *                        (may alias residual_in), out = RMSNorm(h)
 * x [T][H] of x_dtype; residual_in/out [T][H] fp32; gamma [H] and out [T][H]
 * of out_dtype.  T may be 0.
 */
dl_status dl_rmsnorm_residual(const void* x, dl_dtype x_dtype, const float* residual_in,
                              float* residual_out, const void* gamma, void* out, int32_t T,
                              int32_t H, float eps, dl_dtype out_dtype, void* stream);

/*
 * Merged QKV projection with the rotary embedding as its epilogue
 * (ops-transformer page, "single-layer operator call chain": MergedMatMul of
 * the three linears sharing x, RoPE applied on the QKV output on chip).
 *   [q | k | v] = x [Wq; Wk; Wv]^T, then q and k of every head rotated at the
 *   token's position with cos_sin (from dl_rope_table_fill).
 * x [T][H]; w_q [Hq*D][H]; w_k, w_v [Hkv*D][H]; positions [T] int32 in
 * [0, max_pos); q [T][Hq][D]; k, v [T][Hkv][D].  All of dtype dt.
 */
size_t dl_qkv_rope_workspace_size(int32_t T, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                                  dl_dtype dt);
dl_status dl_qkv_rope(const void* x, const void* w_q, const void* w_k, const void* w_v,
                      const int32_t* positions, const float* cos_sin, int32_t max_pos, void* q,
                      void* k, void* v, int32_t T, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                      dl_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * QKV + RoPE with the reshape-and-cache write fused into the epilogue (the KV
 * update folded into the attention block: ascend-transformer-boost fusion
 * page, section "KVCache management"; ATB KV-cache page, "KV cache memory
 * bottleneck").  Computes what dl_qkv_rope computes and also writes the
 * rotated k and v of token t to the caches exactly as dl_reshape_and_cache
 * would (same bits): sequence seq_of_token[t] (t itself when NULL), block
 * block_table[seq][positions[t] / BS], slot positions[t] % BS.  k and v may
 * both be NULL (then they go to the cache only) or both be given.  Table
 * entries outside [0, num_blocks) and positions outside the table are
 * skipped.  Workspace as dl_qkv_rope_workspace_size.  DL_KV_LAYER caches
 * only (an INT8 cache returns DL_ERR_UNSUPPORTED; write it with dl_qkv_rope
 * followed by dl_reshape_and_cache).
 */
dl_status dl_qkv_rope_cache(const void* x, const void* w_q, const void* w_k, const void* w_v,
                            const int32_t* positions, const float* cos_sin, int32_t max_pos,
                            void* q, void* k, void* v, const int32_t* seq_of_token,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const dl_kv_cache* cache, int32_t T, int32_t H, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t BS, dl_dtype dt, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Reshape-and-cache (ATB KV-cache page, "KV cache memory bottleneck":
 * ReshapeAndCache writes step K/V into the paged blocks through block_table).
 * Token t of sequence seq_of_token[t] at position positions[t] is copied to
 * block block_table[seq][pos / BS], slot pos % BS, of both caches.  A bit
 * copy for a DL_KV_LAYER cache; a DL_KV_INT8 cache gets each (token, kv
 * head) row of k and of v quantised as dl_kv_format describes, its scale
 * going to the same (block, head, slot) of k_scale / v_scale.  k, v
 * [T][Hkv][D] of dtype dt; seq_of_token [T] int32, or NULL meaning
 * seq_of_token[t] = t (one token per sequence, the decode case).  Table
 * entries outside [0, num_blocks) drop the token's write.
 */
dl_status dl_reshape_and_cache(const void* k, const void* v, const int32_t* seq_of_token,
                               const int32_t* positions, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const dl_kv_cache* cache, int32_t T,
                               int32_t Hkv, int32_t D, int32_t BS, dl_dtype dt, void* stream);

/*
 * Prefill attention: causal, variable-length, grouped-query flash attention
 * (ATB fusion-strategy page, "Attention fusion"; ops-transformer page, "KV
 * cache and operators": prefill sends the full sequence through
 * FlashAttention).  Packed sequences: sequence b owns rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens [B+1] int32, device, with
 * cu_seqlens[B] == T and every length <= max_seqlen).  Row i of a sequence
 * attends to rows 0..i of the same sequence; kv head = h / (Hq/Hkv).
 * q, out [T][Hq][D]; k, v [T][Hkv][D].  scale multiplies q.k before the
 * softmax; scale <= 0 selects 1/sqrt(D), the scaled dot-product of the
 * pages (ATB decoder-layer page, "operator fusion graph of a decoder layer").
 */
dl_status dl_attn_prefill(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t max_seqlen,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, void* out, dl_dtype dt,
                          void* stream);

/*
 * Paged decode attention (ops-transformer page, "KV cache and operators":
 * Q [1, heads, 1, dim] against cached K/V with a decode-specialised kernel;
 * ATB KV-cache page: PagedAttention over block_table and contextLens).
 * Sequence b attends over cached positions 0 .. context_lens[b]-1 (the new
 * token must already be in the cache).  q, out [B][Hq][D].  The result does
 * not depend on which physical blocks hold the data.  A DL_KV_INT8 cache is
 * dequantised (code x row scale) as its blocks are read.  scale <= 0 selects
 * 1/sqrt(D), as for dl_attn_prefill.
 */
size_t dl_attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                     int32_t max_context_len, int32_t BS);
dl_status dl_attn_decode_paged(const void* q, const dl_kv_cache* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len, int32_t B,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, float scale,
                               void* out, dl_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * dl_attn_decode_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with the split
 * partials kept in a fixed device scratch array of the library instead of a
 * caller workspace.  Nothing is allocated per call (no hipMalloc, hipFree or
 * allocating library routine).  The scratch holds
 * dl_attn_decode_noalloc_max_scratch() = 32 MiB on every GPU the library
 * runs on, from load until the process ends; a call whose
 * dl_attn_decode_workspace_size exceeds it returns DL_ERR_WORKSPACE and
 * enqueues nothing.  Every call on one GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (different streams, or host threads
 * enqueueing concurrently) race; calls on one stream are ordered and safe.
 * The scratch needs no clearing: every partial a call reads it wrote first.
 */
dl_status dl_attn_decode_paged_noalloc(const void* q, const dl_kv_cache* cache,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                                       float scale, void* out, dl_dtype dt, void* stream);
size_t dl_attn_decode_noalloc_max_scratch(void);

/*
 * Paged attention for several new tokens per sequence (ATB KV-cache page,
 * section "speculative decoding": the paged attention verifies every
 * sequence's candidate tokens in one pass, with per-sequence query lengths
 * qLens and context lengths contextLens).  Sequence b brings q_len_b =
 * cu_q_lens[b+1] - cu_q_lens[b] query tokens (q, out [Tq][Hq][D] packed in
 * that order, cu_q_lens [B+1] int32 with cu_q_lens[B] == Tq, every q_len_b
 * <= max_q_len); they are the last q_len_b of its context_lens[b] cached
 * positions (written before the call), and new token i, at position
 * context_lens[b] - q_len_b + i, attends over cached positions 0 .. its own
 * (causal among the new tokens).  q_len 1 everywhere is dl_attn_decode_paged;
 * q_len = context_lens is a prefill that reads its keys from the cache; a
 * q_len of 0 is allowed.  Preconditions as for dl_attn_decode_paged, plus
 * q_len_b <= context_lens[b] <= max_context_len.  Layer-dtype caches only
 * (an INT8 cache returns DL_ERR_UNSUPPORTED).  scale <= 0 selects 1/sqrt(D).
 */
size_t dl_attn_paged_qlens_workspace_size(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                                          int32_t D, int32_t max_q_len,
                                          int32_t max_context_len, int32_t BS);
dl_status dl_attn_paged_qlens(const void* q, const dl_kv_cache* cache, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                              const int32_t* context_lens, int32_t B, int32_t Tq,
                              int32_t max_q_len, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t BS, float scale, void* out, dl_dtype dt,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * Plain projection out = x W^T (the attention output linear of the chain,
 * exported for step-by-step use).  x [M][K], w [N][K], out [M][N], dtype dt.
 */
size_t dl_linear_workspace_size(int32_t M, int32_t N, int32_t K, dl_dtype dt);
dl_status dl_linear(const void* x, const void* w, void* out, int32_t M, int32_t N, int32_t K,
                    dl_dtype dt, void* ws, size_t ws_bytes, void* stream);

/*
 * SwiGLU feed-forward with the residual add fused into the down projection
 * (ops-transformer page: MergedMatMul(GateUp), SiLU, gate x up, down linear;
 * ATB fusion-strategy page, "MLP fusion": residual fused into the last dense).
 *   a   = silu(x Wg^T) * (x Wu^T)          (stage 1, a kept in the workspace)
 *   out = residual + a Wd^T                 (stage 2; residual may be NULL)
 * x [T][H] dtype dt; w_gate, w_up [I][H]; w_down [H][I]; residual, out [T][H]
 * fp32 (out may alias residual).
 */
size_t dl_ffn_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt);
dl_status dl_ffn_swiglu(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                        const float* residual, float* out, int32_t T, int32_t H, int32_t I,
                        dl_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* Stage 1 alone: a [T][I] (dtype dt) = silu(x Wg^T) * (x Wu^T). */
size_t dl_gate_up_silu_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt);
dl_status dl_gate_up_silu(const void* x, const void* w_gate, const void* w_up, void* a, int32_t T,
                          int32_t H, int32_t I, dl_dtype dt, void* ws, size_t ws_bytes,
                          void* stream);

/* Stage 2 alone: out [T][H] fp32 = residual + a Wd^T (residual may be NULL). */
size_t dl_down_residual_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt);
dl_status dl_down_residual(const void* a, const void* w_down, const float* residual, float* out,
                           int32_t T, int32_t H, int32_t I, dl_dtype dt, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Whole layer.  Workspace for any call with T <= max_tokens, B <= max_batch,
 * every prefill length <= max_seqlen and every decode context length <=
 * max_context_len.
 */
size_t dl_layer_workspace_size(const dl_layer_dims* d, int32_t max_tokens, int32_t max_batch,
                               int32_t max_seqlen, int32_t max_context_len, dl_mode m);

/*
 * Prefill of B packed sequences (T tokens in total).
 *   hidden_in [T][H] fp32 -> hidden_out [T][H] fp32 (must not alias).
 *   positions [T] (restart at 0 in every sequence), seq_of_token [T],
 *   cu_seqlens [B+1]; every token's K/V is also written to the cache.
 * Attention reads K/V straight from the projection output.  DL_KV_INT8
 * caches need m == DL_FUSED (the kernel-per-op chain is the baseline of the
 * layer-dtype cache; it returns DL_ERR_UNSUPPORTED for them).
 */
dl_status dl_layer_prefill(const dl_layer_dims* d, const dl_layer_weights* w,
                           const float* cos_sin, int32_t max_pos, const float* hidden_in,
                           float* hidden_out, const int32_t* positions,
                           const int32_t* seq_of_token, const int32_t* cu_seqlens, int32_t B,
                           int32_t T, int32_t max_seqlen, const dl_kv_cache* cache,
                           const int32_t* block_table, int32_t max_blocks_per_seq, dl_mode m,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step: one new token per sequence.
 *   hidden_in [B][H] fp32 -> hidden_out [B][H] fp32 (must not alias);
 *   positions [B] = context_lens - 1; context_lens [B] counts the new token.
 * The new K/V are written to the cache first, then attention runs over the
 * whole cached context (ascend-transformer-boost page, "KVCache management":
 * update the cache in place, then attend over the full cache).  DL_KV_INT8
 * caches need m == DL_FUSED, as for dl_layer_prefill.
 */
dl_status dl_layer_decode(const dl_layer_dims* d, const dl_layer_weights* w,
                          const float* cos_sin, int32_t max_pos, const float* hidden_in,
                          float* hidden_out, const int32_t* positions,
                          const int32_t* context_lens, int32_t max_context_len, int32_t B,
                          const dl_kv_cache* cache, const int32_t* block_table,
                          int32_t max_blocks_per_seq, dl_mode m, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * One step that brings q_len_b new tokens to each of B cached sequences:
 * speculative verification of candidate tokens, or a chunk of a prefill over
 * a cached prefix (ATB KV-cache page, section "speculative decoding": the
 * target model's layers run the candidates of all sequences in one pass with
 * PagedAttention given qLens and contextLens).
 *   hidden_in [T][H] fp32 -> hidden_out [T][H] fp32 (must not alias), T =
 *   sum of q_len_b, packed by cu_q_lens [B+1]; seq_of_token [T];
 *   positions [T] = context_lens[b] - q_len_b + i for new token i;
 *   context_lens [B] count the new tokens.
 * The new K/V are written to the cache first; attention is
 * dl_attn_paged_qlens over the cache; the rest is the prefill layer.
 * DL_FUSED and layer-dtype caches only.  Workspace from
 * dl_layer_decode_qlens_workspace_size (T <= max_tokens, B <= max_batch,
 * q_len_b <= max_q_len, context_lens <= max_context_len).
 */
size_t dl_layer_decode_qlens_workspace_size(const dl_layer_dims* d, int32_t max_tokens,
                                            int32_t max_batch, int32_t max_q_len,
                                            int32_t max_context_len);
dl_status dl_layer_decode_qlens(const dl_layer_dims* d, const dl_layer_weights* w,
                                const float* cos_sin, int32_t max_pos, const float* hidden_in,
                                float* hidden_out, const int32_t* positions,
                                const int32_t* seq_of_token, const int32_t* cu_q_lens,
                                const int32_t* context_lens, int32_t B, int32_t T,
                                int32_t max_q_len, int32_t max_context_len,
                                const dl_kv_cache* cache, const int32_t* block_table,
                                int32_t max_blocks_per_seq, dl_mode m, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * A decode step recorded once as a HIP graph and replayed per step, so the
 * step's 9-13 kernels go to the GPU in one launch with no host gaps between
 * them (ATB KV-cache page, section "KV cache memory bottleneck": the
 * GraphOpBuilder groups ReshapeAndCache and PagedAttention into one graph
 * operation so no stream bubble opens between them; ATB decoder-layer page,
 * "graph execution engine").
 *
 * dl_layer_decode_graph_create records dl_layer_decode with exactly these
 * arguments on `stream` (which must not be NULL: the legacy default stream
 * cannot be captured) and instantiates it.  Nothing runs during creation.
 * Every pointer is baked into the graph: between replays the caller rewrites
 * the CONTENTS of hidden_in, positions and context_lens (and of the caches
 * and block_table) in place; B is fixed, and every context length must stay
 * <= the max_context_len given here (the launch grids are sized for it).
 * dl_graph_launch replays it on any stream; dl_graph_destroy frees the
 * host-side graph objects.  The graph holds no device memory of its own.
 * Errors: those of dl_layer_decode (nothing recorded, *graph untouched), or
 * DL_ERR_HIP if capture or instantiation fails.
 */
/*
 * Validation of the index inputs of the paged-cache calls (the ReshapeAndCache
 * and PagedAttention inputs of the ATB KV-cache page, section "KV cache memory
 * bottleneck": block_table, positions, the token's sequence, contextLens; and
 * the packed-sequence offsets of prefill).  Enqueues one small kernel that
 * reads the given arrays and stores into *error_word (device int32, 4-byte
 * aligned; overwritten, no clearing needed) the OR of one bit per violated
 * device-side precondition listed at the top of this header:
 *   DL_CHECK_BIT_SEQ       seq_of_token[t] outside [0, B)
 *   DL_CHECK_BIT_POSITION  positions[t] outside [0, max_blocks_per_seq * BS)
 *   DL_CHECK_BIT_BLOCK     a table entry some token writes, or some context
 *                          position reads, outside [0, num_blocks)
 *   DL_CHECK_BIT_CONTEXT   context_lens[b] outside [1, max_context_len] or
 *                          beyond max_blocks_per_seq * BS
 *   DL_CHECK_BIT_CU        cu_seqlens not 0 .. T nondecreasing, or a length
 *                          above max_seqlen
 * 0 means every given array is valid.  Any array may be NULL to skip its
 * checks (seq_of_token NULL means seq_of_token[t] = t, the decode case).
 * block_table [B][max_blocks_per_seq]; positions, seq_of_token [T];
 * context_lens [B]; cu_seqlens [B+1].  It is a debug aid: the compute calls
 * keep their own clamps, so nothing here is needed for memory safety.
 */
enum {
  DL_CHECK_BIT_SEQ = 1,
  DL_CHECK_BIT_POSITION = 2,
  DL_CHECK_BIT_BLOCK = 4,
  DL_CHECK_BIT_CONTEXT = 8,
  DL_CHECK_BIT_CU = 16
};
dl_status dl_check_indices(const int32_t* block_table, int32_t B, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t BS, const int32_t* positions,
                           const int32_t* seq_of_token, int32_t T, const int32_t* context_lens,
                           int32_t max_context_len, const int32_t* cu_seqlens,
                           int32_t max_seqlen, int32_t* error_word, void* stream);

/*
 * Named regions of a layer workspace, for inspecting a call's intermediates
 * after it ran: the debugging method of the ATB fusion-strategy page (section
 * "debugging"), which runs the chain step by step and compares each
 * intermediate tensor with the fused result.  After dl_layer_prefill (or
 * dl_layer_decode) returns and its stream has finished, the workspace holds
 * that call's intermediates until the next call that uses it:
 *   DL_WS_N1, DL_WS_N2    normalised activations [T][H] (dtype)
 *   DL_WS_Q, DL_WS_K, DL_WS_V   q [T][Hq][D], k, v [T][Hkv][D] after RoPE
 *                         (the fused decode step with a layer-dtype cache
 *                         writes k/v to the cache only, so there they are
 *                         not filled)
 *   DL_WS_ATTN            attention output [T][Hq*D]
 *   DL_WS_O               output projection [T][H]
 *   DL_WS_H               residual stream after attention [T][H] fp32
 *   DL_WS_A               silu(gate) * up [T][I]
 *   DL_UNFUSED only:      DL_WS_SCORES fp32 [B][Hq][S][S] (prefill, S =
 *                         max_seqlen, -inf above the diagonal) or [B][Hq][S]
 *                         (decode, S = max_context_len); DL_WS_PROBS the
 *                         softmax of each row (dtype), same shape;
 *                         DL_WS_GATE, DL_WS_UP, DL_WS_SILU [T][I] (dtype);
 *                         DL_WS_DOWN the down projection [T][H] fp32
 *   DL_WS_PARTIAL, DL_WS_DECODE   GEMM and attention split partials (opaque)
 * offsets[r] and sizes[r] (host arrays of DL_WS_COUNT) receive each region's
 * byte offset into the workspace and its byte size (0 when the call does not
 * use it).  is_decode 0: the prefill layout for (T, B, max_seqlen); 1: the
 * decode layout for (B, max_context_len), with T == B.  The dims and sizes
 * are checked as the layer calls check them.
 */
typedef enum {
  DL_WS_N1 = 0, DL_WS_Q, DL_WS_K, DL_WS_V, DL_WS_ATTN, DL_WS_O, DL_WS_H, DL_WS_N2, DL_WS_A,
  DL_WS_PARTIAL, DL_WS_DECODE, DL_WS_SCORES, DL_WS_PROBS, DL_WS_GATE, DL_WS_UP, DL_WS_SILU,
  DL_WS_DOWN, DL_WS_COUNT
} dl_ws_region;
dl_status dl_layer_workspace_regions(const dl_layer_dims* d, int32_t T, int32_t B,
                                     int32_t max_seqlen_or_context, int32_t is_decode, dl_mode m,
                                     size_t* offsets, size_t* sizes);

typedef struct dl_graph_s* dl_graph;
dl_status dl_layer_decode_graph_create(const dl_layer_dims* d, const dl_layer_weights* w,
                                       const float* cos_sin, int32_t max_pos,
                                       const float* hidden_in, float* hidden_out,
                                       const int32_t* positions, const int32_t* context_lens,
                                       int32_t max_context_len, int32_t B,
                                       const dl_kv_cache* cache, const int32_t* block_table,
                                       int32_t max_blocks_per_seq, void* ws, size_t ws_bytes,
                                       void* stream, dl_graph* graph);
dl_status dl_graph_launch(dl_graph graph, void* stream);
dl_status dl_graph_destroy(dl_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* DL_LAYER_H */
