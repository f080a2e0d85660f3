/*
 * orc.c -- CPU oracle for the Llama-style decoder-layer forward (prefill and
 * paged decode).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no source with the HIP library.
 *
 * Conventions
 *   - every tensor is a dense row-major fp32 array (bf16 data is held as the
 *     fp32 value it represents);
 *   - every dot product and every reduction accumulates in fp64, in plain
 *     index order, and the result is rounded once to fp32 when it is stored;
 *   - weights are [out_features][in_features]; a linear layer is y = x W^T.
 *
 * Rounding modes (a switch on where results are stored, not a second
 * algorithm):
 *   ORC_EXACT          fp32 storage everywhere;
 *   ORC_BF16           fp32 -> bf16 round-to-nearest-even at the tensors the
 *                      fused GPU path stores in bf16: n1, rotated q/k, v
 *                      (hence the cache), attention output, o, n2, a.  The
 *                      residual stream (x, h, y) stays fp32;
 *   ORC_BF16_UNFUSED   ORC_BF16 plus the extra storage points of a
 *                      kernel-per-op chain: q/k before rotation, gate, up,
 *                      silu(gate) and the softmax probabilities P (scores S
 *                      stay fp32).
 *
 * Sources (the pages are cited by site and section):
 *   [chain]  ops-transformer Llama2-7B operator page (seekfood.cn), paragraph
 *            "single-layer operator call chain": x -> RMSNorm -> Q/K/V linear
 *            -> rotary embedding -> self-attention (GQA) -> output linear ->
 *            residual -> RMSNorm -> gate/up linear -> SiLU -> down linear ->
 *            residual;  paragraph "KV cache and operators": prefill runs the
 *            full sequence through attention, decode has one query row and
 *            reads K/V from the cache.
 *   [graph]  ATB decoder-layer page (ai6s.net), section "operator fusion
 *            graph of a decoder layer": Input -> Norm1 -> Attention -> Add ->
 *            Norm2 -> FFN -> Add, attention = QKV projection -> scaled
 *            dot-product -> softmax -> output projection.
 *   [kvpage] ATB KV-cache page (hwcomputing.csdn.net), section "KV cache
 *            memory bottleneck": fixed-size blocks addressed through
 *            block_table, contextLens growing per step, ReshapeAndCache
 *            writing step K/V into the blocks.
 *   [kvupd]  ascend-transformer-boost fusion page (agent.csdn.net), section
 *            "KVCache management": compute new K/V, update the cache in
 *            place, then attend over the whole cache.
 *   [ffn]    same page, section "fusion operator matrix": FFN weights
 *            w_gate, w_up [intermediate, hidden], w_down [hidden,
 *            intermediate]; norm fused with the residual add.
 *   [mlp]    ATB fusion-strategy page (gitcode.csdn.net), section "MLP
 *            fusion": residual add fused into the last dense layer; section
 *            "configuration": LLaMA uses SiLU.
 *   [spec]   ATB KV-cache page, section "speculative decoding": the paged
 *            attention verifies K candidate tokens of a sequence in one
 *            pass, qLens giving each sequence's number of query tokens and
 *            contextLens its cached length.
 *   [kvquant] ATB KV-cache page (hwcomputing.csdn.net), section "KV cache
 *            quantisation (INT8/INT4 precision-latency trade-off)": at
 *            per-token granularity each token's K and its V carry their own
 *            fp32 scale; online quantisation computes the scale as the token
 *            is written; PagedAttention dequantises while it loads cache
 *            blocks; the scales sit in HBM beside the blocks.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   RMSNorm in the Llama form (eps inside the root, gamma after normalising);
 *   rotate-half RoPE pairing (i, i + D/2) with w_i = theta^(-2i/D), angles in
 *   fp64 (the pages give no rotary formula); attention scale 1/sqrt(D);
 *   GQA kv head = q head div (Hq/Hkv); SwiGLU a = silu(gate) * up;
 *   decode writes the new token to the cache before attending, and
 *   context_lens counts that token;
 *   several new tokens per sequence (qLens): they are the last q_len
 *   positions of the cache, written before attending, and each sees the
 *   positions up to its own (causal among the new tokens, as in prefill);
 *   INT8 KV rows: symmetric (no offset), one scale per (token, kv head) row
 *   of K and of V, scale = max|x| / 127, code = x / scale rounded to the
 *   nearest integer (ties to even) and clamped to [-127, 127], both in fp32
 *   (the precision the page gives the scale); an all-zero row has scale 0
 *   and codes 0; a dequantised element is code x scale.
 *
 * Parity pins: every function here is pinned by CPU tests against closed
 * forms, invariants, exact integer cases and brute force (tests/test_oracle_*).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXACT 0
#define ORC_BF16 1
#define ORC_BF16_UNFUSED 2

/* ------------------------------------------------------------------------ */
/* bf16 storage emulation                                                    */
/* ------------------------------------------------------------------------ */

/* fp32 -> bf16 -> fp32, round to nearest, ties to even; NaN stays NaN. */
float orc_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    u = (u | 0x00400000u) & 0xffff0000u; /* quiet NaN, sign kept */
  } else {
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7fffu + lsb) & 0xffff0000u;
  }
  float r;
  memcpy(&r, &u, 4);
  return r;
}

void orc_round_bf16_array(float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_bf16_round(x[i]);
}

static inline float store(double v, int round_bf16) {
  float f = (float)v;
  return round_bf16 ? orc_bf16_round(f) : f;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm, optionally after the residual add   [chain], [graph], [ffn]      */
/* ------------------------------------------------------------------------ */

/*
 * If resid_in is NULL:  out = gamma * x / sqrt(mean(x^2) + eps).
 * Otherwise:            h = x + resid_in (one fp32 add, written to
 *                       resid_out), out = gamma * h / sqrt(mean(h^2) + eps).
 * out is rounded to bf16 when mode != ORC_EXACT.
 */
void orc_rmsnorm(const float* x, const float* resid_in, float* resid_out,
                 const float* gamma, float* out, int T, int H, double eps,
                 int mode) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (int64_t)t * H;
    float* hr = NULL;
    if (resid_in) {
      hr = resid_out + (int64_t)t * H;
      const float* rr = resid_in + (int64_t)t * H;
      for (int i = 0; i < H; ++i) hr[i] = (float)((double)xr[i] + (double)rr[i]);
      xr = hr;
    }
    double ss = 0.0;
    for (int i = 0; i < H; ++i) ss += (double)xr[i] * (double)xr[i];
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    float* o = out + (int64_t)t * H;
    for (int i = 0; i < H; ++i)
      o[i] = store((double)gamma[i] * ((double)xr[i] * inv), mode != ORC_EXACT);
  }
}

/* ------------------------------------------------------------------------ */
/* Linear layer y = x W^T                                                    */
/* ------------------------------------------------------------------------ */

/* x [M][K], W [N][K] -> y [M][N]; fp64 accumulation in k order. */
void orc_linear(const float* x, const float* W, float* y, int M, int N, int K,
                int round_bf16) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      const float* xr = x + (int64_t)m * K;
      const float* wr = W + (int64_t)n * K;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += (double)xr[k] * (double)wr[k];
      y[(int64_t)m * N + n] = store(acc, round_bf16);
    }
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding (rotate-half pairing)                [chain]   */
/* ------------------------------------------------------------------------ */

/*
 * u [T][nh][D] rotated in place at positions pos[T]:
 *   for i < D/2:  phi = pos * theta^(-2i/D)   (fp64)
 *     u'[i]       = u[i] cos(phi) - u[i+D/2] sin(phi)
 *     u'[i+D/2]   = u[i+D/2] cos(phi) + u[i] sin(phi)
 */
void orc_rope(float* u, const int32_t* pos, int T, int nh, int D, double theta,
              int round_bf16) {
  const int half = D / 2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < nh; ++h) {
      float* v = u + ((int64_t)t * nh + h) * D;
      for (int i = 0; i < half; ++i) {
        double w = pow(theta, -2.0 * (double)i / (double)D);
        double phi = (double)pos[t] * w;
        double c = cos(phi), s = sin(phi);
        double a = v[i], b = v[i + half];
        v[i] = store(a * c - b * s, round_bf16);
        v[i + half] = store(b * c + a * s, round_bf16);
      }
    }
}

/*
 * Merged QKV projection followed by RoPE on q and k             [chain]
 * x [T][H]; Wq [Hq*D][H], Wk/Wv [Hkv*D][H]; q [T][Hq][D], k/v [T][Hkv][D].
 */
void orc_qkv_rope(const float* x, const float* wq, const float* wk,
                  const float* wv, const int32_t* pos, double theta, float* q,
                  float* k, float* v, int T, int H, int Hq, int Hkv, int D,
                  int mode) {
  const int pre_round = (mode == ORC_BF16_UNFUSED);
  orc_linear(x, wq, q, T, Hq * D, H, pre_round);
  orc_linear(x, wk, k, T, Hkv * D, H, pre_round);
  orc_linear(x, wv, v, T, Hkv * D, H, mode != ORC_EXACT);
  orc_rope(q, pos, T, Hq, D, theta, mode != ORC_EXACT);
  orc_rope(k, pos, T, Hkv, D, theta, mode != ORC_EXACT);
}

/* ------------------------------------------------------------------------ */
/* Reshape-and-cache into block_table-addressed blocks            [kvpage]  */
/* ------------------------------------------------------------------------ */

/*
 * Cache layout: [num_blocks][Hkv][BS][D].  Token t of sequence s at position
 * p lands in physical block block_table[s][p / BS], slot p % BS.  A copy.
 */
void orc_reshape_and_cache(const float* k, const float* v,
                           const int32_t* seq_of_token, const int32_t* pos,
                           const int32_t* block_table, int max_blocks_per_seq,
                           float* k_cache, float* v_cache, int T, int Hkv,
                           int D, int BS) {
  for (int t = 0; t < T; ++t) {
    int s = seq_of_token[t], p = pos[t];
    int blk = block_table[(int64_t)s * max_blocks_per_seq + p / BS];
    int slot = p % BS;
    for (int g = 0; g < Hkv; ++g) {
      int64_t dst = (((int64_t)blk * Hkv + g) * BS + slot) * D;
      int64_t src = ((int64_t)t * Hkv + g) * D;
      memcpy(k_cache + dst, k + src, sizeof(float) * (size_t)D);
      memcpy(v_cache + dst, v + src, sizeof(float) * (size_t)D);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Attention core: softmax(q.K^T * scale) V over an explicit key list        */
/* ------------------------------------------------------------------------ */

/*
 * keys[j], vals[j] point at D-vectors; n keys.  o = sum_j P_j v_j with
 * P = softmax(s), s_j = scale * q.k_j, max subtracted.  In the unfused mode
 * the scores are stored in fp32 and P in bf16 before the PV product.
 * kmul / vmul (NULL = all ones) multiply every element of key j / value j:
 * an INT8 row is passed as its codes with its scale as the multiplier, so
 * the element used is the dequantised code x scale (an exact product in
 * fp64).  scratch holds n doubles.
 */
static void attend_keep(const float* q, const float* const* keys,
                        const float* const* vals, const double* kmul,
                        const double* vmul, int n, int D, double scale,
                        float* out, int mode, double* s, float* s_keep,
                        float* p_keep) {
  double mx = -INFINITY;
  for (int j = 0; j < n; ++j) {
    const double km = kmul ? kmul[j] : 1.0;
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += (double)q[d] * ((double)keys[j][d] * km);
    s[j] = acc * scale;
    if (mode == ORC_BF16_UNFUSED) s[j] = (double)(float)s[j];
    if (s_keep) s_keep[j] = (float)s[j];
    if (s[j] > mx) mx = s[j];
  }
  double l = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - mx);
    l += s[j];
  }
  for (int j = 0; j < n; ++j) {
    s[j] /= l;
    if (mode == ORC_BF16_UNFUSED) s[j] = (double)orc_bf16_round((float)s[j]);
    if (p_keep) p_keep[j] = (float)s[j];
  }
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j)
      acc += s[j] * ((double)vals[j][d] * (vmul ? vmul[j] : 1.0));
    out[d] = store(acc, mode != ORC_EXACT);
  }
}

static void attend(const float* q, const float* const* keys,
                   const float* const* vals, const double* kmul,
                   const double* vmul, int n, int D, double scale, float* out,
                   int mode, double* s) {
  attend_keep(q, keys, vals, kmul, vmul, n, D, scale, out, mode, s, NULL, NULL);
}

/*
 * One query row over n contiguous keys k [n][D] and values v [n][D]: the
 * same computation as every attention function here, with its scores and
 * probabilities also returned as the kernel-per-op chain stores them
 * (s_out: fp32 scores after the scale; p_out: probabilities, bf16 in
 * ORC_BF16_UNFUSED).  o [D] is the row's output.             [chain]
 */
void orc_attn_row(const float* q, const float* k, const float* v, int n, int D,
                  double scale, int mode, float* s_out, float* p_out,
                  float* o) {
  const float** keys = (const float**)malloc(sizeof(float*) * (size_t)(n > 0 ? n : 1));
  const float** vals = (const float**)malloc(sizeof(float*) * (size_t)(n > 0 ? n : 1));
  double* sc = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int j = 0; j < n; ++j) {
    keys[j] = k + (int64_t)j * D;
    vals[j] = v + (int64_t)j * D;
  }
  attend_keep(q, keys, vals, NULL, NULL, n, D, scale, o, mode, sc, s_out, p_out);
  free(keys);
  free(vals);
  free(sc);
}

/*
 * Causal varlen prefill attention with GQA                [chain], [graph]
 * Packed tokens: sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1.
 * q [T][Hq][D], k/v [T][Hkv][D] -> out [T][Hq][D].  Query i of a sequence
 * sees keys 0..i of the same sequence; kv head g = h / (Hq/Hkv).
 */
void orc_attn_prefill(const float* q, const float* k, const float* v,
                      const int32_t* cu_seqlens, int B, int Hq, int Hkv, int D,
                      double scale, float* out, int mode) {
  const int grp = Hq / Hkv;
  for (int b = 0; b < B; ++b) {
    const int t0 = cu_seqlens[b], S = cu_seqlens[b + 1] - cu_seqlens[b];
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int i = 0; i < S; ++i)
      for (int h = 0; h < Hq; ++h) {
        const int g = h / grp;
        const float** keys = (const float**)malloc(sizeof(float*) * (size_t)(i + 1));
        const float** vals = (const float**)malloc(sizeof(float*) * (size_t)(i + 1));
        double* sc = (double*)malloc(sizeof(double) * (size_t)(i + 1));
        for (int j = 0; j <= i; ++j) {
          keys[j] = k + ((int64_t)(t0 + j) * Hkv + g) * D;
          vals[j] = v + ((int64_t)(t0 + j) * Hkv + g) * D;
        }
        attend(q + ((int64_t)(t0 + i) * Hq + h) * D, keys, vals, NULL, NULL, i + 1, D, scale,
               out + ((int64_t)(t0 + i) * Hq + h) * D, mode, sc);
        free(keys);
        free(vals);
        free(sc);
      }
  }
}

/*
 * Paged decode attention                               [chain], [kvpage]
 * q [B][Hq][D] (one new token per sequence); the cache already holds that
 * token.  Sequence b attends over logical positions 0 .. ctx_b - 1, position
 * j living in block block_table[b][j / BS], slot j % BS.
 */
void orc_attn_decode_paged(const float* q, const float* k_cache,
                           const float* v_cache, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* context_lens,
                           int B, int Hq, int Hkv, int D, int BS, double scale,
                           float* out, int mode) {
  const int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h) {
      const int g = h / grp, n = context_lens[b];
      const float** keys = (const float**)malloc(sizeof(float*) * (size_t)n);
      const float** vals = (const float**)malloc(sizeof(float*) * (size_t)n);
      double* sc = (double*)malloc(sizeof(double) * (size_t)n);
      for (int j = 0; j < n; ++j) {
        int blk = block_table[(int64_t)b * max_blocks_per_seq + j / BS];
        int64_t off = (((int64_t)blk * Hkv + g) * BS + j % BS) * D;
        keys[j] = k_cache + off;
        vals[j] = v_cache + off;
      }
      attend(q + ((int64_t)b * Hq + h) * D, keys, vals, NULL, NULL, n, D, scale,
             out + ((int64_t)b * Hq + h) * D, mode, sc);
      free(keys);
      free(vals);
      free(sc);
    }
}

/*
 * Paged attention for several new query tokens per sequence   [kvpage], [spec]
 * Sequence b brings q_len_b = cu_q[b+1] - cu_q[b] query rows (packed in q
 * [Tq][Hq][D]); its cache already holds all ctx_b = context_lens[b]
 * positions, the new tokens being the last q_len_b of them.  New token i
 * sits at position p_i = ctx_b - q_len_b + i and attends over the cached
 * positions 0 .. p_i (the earlier new tokens included, the later ones not).
 * q_len_b = 1 is the decode step.
 */
void orc_attn_paged_qlens(const float* q, const float* k_cache,
                          const float* v_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* cu_q,
                          const int32_t* context_lens, int B, int Hq, int Hkv,
                          int D, int BS, double scale, float* out, int mode) {
  const int grp = Hq / Hkv;
  for (int b = 0; b < B; ++b) {
    const int q0 = cu_q[b], ql = cu_q[b + 1] - cu_q[b];
    const int first = context_lens[b] - ql; /* position of the first new token */
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int i = 0; i < ql; ++i)
      for (int h = 0; h < Hq; ++h) {
        const int g = h / grp, n = first + i + 1;
        const float** keys = (const float**)malloc(sizeof(float*) * (size_t)n);
        const float** vals = (const float**)malloc(sizeof(float*) * (size_t)n);
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
        for (int j = 0; j < n; ++j) {
          int blk = block_table[(int64_t)b * max_blocks_per_seq + j / BS];
          int64_t off = (((int64_t)blk * Hkv + g) * BS + j % BS) * D;
          keys[j] = k_cache + off;
          vals[j] = v_cache + off;
        }
        attend(q + ((int64_t)(q0 + i) * Hq + h) * D, keys, vals, NULL, NULL, n, D,
               scale, out + ((int64_t)(q0 + i) * Hq + h) * D, mode, sc);
        free(keys);
        free(vals);
        free(sc);
      }
  }
}

/*
 * Decode attention over a contiguous cache [B][Hkv][S][D]     [kvupd]
 * (the un-paged form of the same computation).
 */
void orc_attn_decode_contig(const float* q, const float* k_cache,
                            const float* v_cache, int S,
                            const int32_t* context_lens, int B, int Hq, int Hkv,
                            int D, double scale, float* out, int mode) {
  const int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h) {
      const int g = h / grp, n = context_lens[b];
      const float** keys = (const float**)malloc(sizeof(float*) * (size_t)n);
      const float** vals = (const float**)malloc(sizeof(float*) * (size_t)n);
      double* sc = (double*)malloc(sizeof(double) * (size_t)n);
      for (int j = 0; j < n; ++j) {
        int64_t off = (((int64_t)b * Hkv + g) * S + j) * D;
        keys[j] = k_cache + off;
        vals[j] = v_cache + off;
      }
      attend(q + ((int64_t)b * Hq + h) * D, keys, vals, NULL, NULL, n, D, scale,
             out + ((int64_t)b * Hq + h) * D, mode, sc);
      free(keys);
      free(vals);
      free(sc);
    }
}

/* ------------------------------------------------------------------------ */
/* SwiGLU feed-forward                                    [chain], [ffn]    */
/* ------------------------------------------------------------------------ */

/*
 * a = silu(x Wg^T) * (x Wu^T), silu(z) = z / (1 + e^-z).  a [M][I].
 * g_out, u_out, sg_out (each [M][I], NULL to skip) receive the gate and up
 * projections and silu(gate) as they are stored (bf16 in ORC_BF16_UNFUSED,
 * the kernel-per-op chain's storage points).
 */
void orc_swiglu_parts(const float* x, const float* wg, const float* wu,
                      float* g_out, float* u_out, float* sg_out, float* a,
                      int M, int H, int I, int mode) {
  const int unf = (mode == ORC_BF16_UNFUSED);
  float* g = g_out ? g_out : (float*)malloc(sizeof(float) * (size_t)M * (size_t)I);
  float* u = u_out ? u_out : (float*)malloc(sizeof(float) * (size_t)M * (size_t)I);
  orc_linear(x, wg, g, M, I, H, unf);
  orc_linear(x, wu, u, M, I, H, unf);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)M * I; ++i) {
    double z = g[i];
    float sl = store(z / (1.0 + exp(-z)), unf);
    if (sg_out) sg_out[i] = sl;
    a[i] = store((double)sl * (double)u[i], mode != ORC_EXACT);
  }
  if (!g_out) free(g);
  if (!u_out) free(u);
}

void orc_swiglu(const float* x, const float* wg, const float* wu, float* a,
                int M, int H, int I, int mode) {
  orc_swiglu_parts(x, wg, wu, NULL, NULL, NULL, a, M, H, I, mode);
}

/* y = resid + a Wd^T (the product is stored in fp32, then one fp32 add). */
void orc_down_residual(const float* a, const float* wd, const float* resid,
                       float* y, int M, int H, int I) {
  orc_linear(a, wd, y, M, H, I, 0);
  if (resid) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)M * H; ++i)
      y[i] = (float)((double)y[i] + (double)resid[i]);
  }
}

/* Whole feed-forward block: y = resid + Wd (silu(Wg x) * Wu x). */
void orc_ffn(const float* x, const float* wg, const float* wu, const float* wd,
             const float* resid, float* y, int M, int H, int I, int mode) {
  float* a = (float*)malloc(sizeof(float) * (size_t)M * (size_t)I);
  orc_swiglu(x, wg, wu, a, M, H, I, mode);
  orc_down_residual(a, wd, resid, y, M, H, I);
  free(a);
}

/* ------------------------------------------------------------------------ */
/* INT8 KV cache with per-token scales, quantised on write      [kvquant]   */
/* ------------------------------------------------------------------------ */

/*
 * One cached row (one token, one kv head, K or V; D values):
 *   scale = max_d |x_d| / 127            (fp32 division)
 *   code_d = nearest integer to x_d / scale, ties to even, in [-127, 127]
 * An all-zero row gets scale 0 and all-zero codes.
 */
void orc_kv_quant_row(const float* x, int D, int8_t* code, float* scale) {
  float amax = 0.0f;
  for (int d = 0; d < D; ++d) {
    float a = fabsf(x[d]);
    if (a > amax) amax = a;
  }
  const float s = amax / 127.0f;
  *scale = s;
  for (int d = 0; d < D; ++d) {
    if (s == 0.0f) {
      code[d] = 0;
      continue;
    }
    float r = rintf(x[d] / s); /* default rounding mode: nearest, ties to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    code[d] = (int8_t)r;
  }
}

/* R consecutive rows of D values (x [R][D] -> codes [R][D], scales [R]). */
void orc_kv_quant_rows(const float* x, int64_t R, int D, int8_t* codes,
                       float* scales) {
  for (int64_t r = 0; r < R; ++r)
    orc_kv_quant_row(x + r * D, D, codes + r * D, scales + r);
}

/*
 * Reshape-and-cache into an INT8 cache: the placement of
 * orc_reshape_and_cache, with each (token, kv head) row of k and of v
 * quantised on the way in.  Codes [num_blocks][Hkv][BS][D] int8; scales
 * [num_blocks][Hkv][BS] fp32, indexed like the rows they belong to.
 */
void orc_reshape_and_cache_q8(const float* k, const float* v,
                              const int32_t* seq_of_token, const int32_t* pos,
                              const int32_t* block_table, int max_blocks_per_seq,
                              int8_t* k_codes, int8_t* v_codes, float* k_scale,
                              float* v_scale, int T, int Hkv, int D, int BS) {
  for (int t = 0; t < T; ++t) {
    int s = seq_of_token[t], p = pos[t];
    int blk = block_table[(int64_t)s * max_blocks_per_seq + p / BS];
    int slot = p % BS;
    for (int g = 0; g < Hkv; ++g) {
      int64_t row = ((int64_t)blk * Hkv + g) * BS + slot;
      int64_t src = ((int64_t)t * Hkv + g) * D;
      orc_kv_quant_row(k + src, D, k_codes + row * D, k_scale + row);
      orc_kv_quant_row(v + src, D, v_codes + row * D, v_scale + row);
    }
  }
}

/*
 * Paged decode attention over an INT8 cache              [kvquant], [kvpage]
 * The computation of orc_attn_decode_paged on the dequantised cache: key j
 * is k_codes row x k_scale of that row, value j likewise (the dequantisation
 * done while the blocks are loaded).
 */
void orc_attn_decode_paged_q8(const float* q, const int8_t* k_codes,
                              const int8_t* v_codes, const float* k_scale,
                              const float* v_scale, const int32_t* block_table,
                              int max_blocks_per_seq, const int32_t* context_lens,
                              int B, int Hq, int Hkv, int D, int BS, double scale,
                              float* out, int mode) {
  const int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h) {
      const int g = h / grp, n = context_lens[b];
      float* kf = (float*)malloc(sizeof(float) * (size_t)n * D);
      float* vf = (float*)malloc(sizeof(float) * (size_t)n * D);
      const float** keys = (const float**)malloc(sizeof(float*) * (size_t)n);
      const float** vals = (const float**)malloc(sizeof(float*) * (size_t)n);
      double* km = (double*)malloc(sizeof(double) * (size_t)n);
      double* vm = (double*)malloc(sizeof(double) * (size_t)n);
      double* sc = (double*)malloc(sizeof(double) * (size_t)n);
      for (int j = 0; j < n; ++j) {
        int blk = block_table[(int64_t)b * max_blocks_per_seq + j / BS];
        int64_t row = ((int64_t)blk * Hkv + g) * BS + j % BS;
        for (int d = 0; d < D; ++d) {  /* codes are integers: exact in fp32 */
          kf[(int64_t)j * D + d] = (float)k_codes[row * D + d];
          vf[(int64_t)j * D + d] = (float)v_codes[row * D + d];
        }
        keys[j] = kf + (int64_t)j * D;
        vals[j] = vf + (int64_t)j * D;
        km[j] = (double)k_scale[row];
        vm[j] = (double)v_scale[row];
      }
      attend(q + ((int64_t)b * Hq + h) * D, keys, vals, km, vm, n, D, scale,
             out + ((int64_t)b * Hq + h) * D, mode, sc);
      free(kf);
      free(vf);
      free(keys);
      free(vals);
      free(km);
      free(vm);
      free(sc);
    }
}

/* ------------------------------------------------------------------------ */
/* Whole decoder layer                            [graph], [chain], [kvupd] */
/* ------------------------------------------------------------------------ */

typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim, intermediate, block_size;
  double rms_eps, rope_theta;
} orc_dims;

typedef struct {
  const float *ln1, *wq, *wk, *wv, *wo, *ln2, *wg, *wu, *wd;
} orc_weights;

/*
 * Tail shared by prefill and decode: o = attn Wo^T, h = x + o,
 * n2 = RMSNorm(h), y = h + FFN(n2).  h is written to h_out when non-NULL.
 */
static void layer_tail(const orc_dims* d, const orc_weights* w, const float* x,
                       const float* attn, float* y, float* h_out, int T,
                       int mode) {
  const int H = d->hidden, Hq = d->n_q_heads, D = d->head_dim, I = d->intermediate;
  float* o = (float*)malloc(sizeof(float) * (size_t)T * H);
  float* h = (float*)malloc(sizeof(float) * (size_t)T * H);
  float* n2 = (float*)malloc(sizeof(float) * (size_t)T * H);
  orc_linear(attn, w->wo, o, T, H, Hq * D, mode != ORC_EXACT);
  orc_rmsnorm(o, x, h, w->ln2, n2, T, H, d->rms_eps, mode);
  orc_ffn(n2, w->wg, w->wu, w->wd, h, y, T, H, I, mode);
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)T * H);
  free(o);
  free(h);
  free(n2);
}

/*
 * Where a layer keeps its K/V: float caches (k, v), or an INT8 cache (codes
 * kq, vq and row scales ks, vs).  Members of the other kind are NULL.
 */
typedef struct {
  float *k, *v;
  int8_t *kq, *vq;
  float *ks, *vs;
} orc_kv;

static void cache_write(const orc_kv* c, const float* k, const float* v,
                        const int32_t* seq, const int32_t* pos,
                        const int32_t* block_table, int max_blocks_per_seq, int T,
                        int Hkv, int D, int BS) {
  if (c->kq)
    orc_reshape_and_cache_q8(k, v, seq, pos, block_table, max_blocks_per_seq,
                             c->kq, c->vq, c->ks, c->vs, T, Hkv, D, BS);
  else if (c->k)
    orc_reshape_and_cache(k, v, seq, pos, block_table, max_blocks_per_seq,
                          c->k, c->v, T, Hkv, D, BS);
}

/*
 * Prefill over packed sequences.  x, y [T][H]; positions restart at 0 in
 * every sequence.  K/V of every token are written to the cache; attention
 * reads k/v straight from the projection output.
 */
static void layer_prefill(const orc_dims* d, const orc_weights* w, const float* x,
                          float* y, float* h_out, const int32_t* pos,
                          const int32_t* seq_of_token, const int32_t* cu_seqlens,
                          int B, int T, const orc_kv* c,
                          const int32_t* block_table, int max_blocks_per_seq,
                          int mode) {
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  float* n1 = (float*)malloc(sizeof(float) * (size_t)T * H);
  float* q = (float*)malloc(sizeof(float) * (size_t)T * Hq * D);
  float* k = (float*)malloc(sizeof(float) * (size_t)T * Hkv * D);
  float* v = (float*)malloc(sizeof(float) * (size_t)T * Hkv * D);
  float* attn = (float*)malloc(sizeof(float) * (size_t)T * Hq * D);
  orc_rmsnorm(x, NULL, NULL, w->ln1, n1, T, H, d->rms_eps, mode);
  orc_qkv_rope(n1, w->wq, w->wk, w->wv, pos, d->rope_theta, q, k, v, T, H, Hq,
               Hkv, D, mode);
  cache_write(c, k, v, seq_of_token, pos, block_table, max_blocks_per_seq, T,
              Hkv, D, d->block_size);
  orc_attn_prefill(q, k, v, cu_seqlens, B, Hq, Hkv, D, 1.0 / sqrt((double)D),
                   attn, mode);
  layer_tail(d, w, x, attn, y, h_out, T, mode);
  free(n1);
  free(q);
  free(k);
  free(v);
  free(attn);
}

/*
 * One decode step: one new token per sequence at position context_lens[b]-1.
 * Its K/V are written into the cache first, then attention runs over the
 * whole cached context (which includes the new token).
 */
static void layer_decode(const orc_dims* d, const orc_weights* w, const float* x,
                         float* y, float* h_out, const int32_t* context_lens,
                         int B, const orc_kv* c, const int32_t* block_table,
                         int max_blocks_per_seq, int mode) {
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  for (int b = 0; b < B; ++b) {
    pos[b] = context_lens[b] - 1;
    seq[b] = b;
  }
  float* n1 = (float*)malloc(sizeof(float) * (size_t)B * H);
  float* q = (float*)malloc(sizeof(float) * (size_t)B * Hq * D);
  float* k = (float*)malloc(sizeof(float) * (size_t)B * Hkv * D);
  float* v = (float*)malloc(sizeof(float) * (size_t)B * Hkv * D);
  float* attn = (float*)malloc(sizeof(float) * (size_t)B * Hq * D);
  const double scale = 1.0 / sqrt((double)D);
  orc_rmsnorm(x, NULL, NULL, w->ln1, n1, B, H, d->rms_eps, mode);
  orc_qkv_rope(n1, w->wq, w->wk, w->wv, pos, d->rope_theta, q, k, v, B, H, Hq,
               Hkv, D, mode);
  cache_write(c, k, v, seq, pos, block_table, max_blocks_per_seq, B, Hkv, D,
              d->block_size);
  if (c->kq)
    orc_attn_decode_paged_q8(q, c->kq, c->vq, c->ks, c->vs, block_table,
                             max_blocks_per_seq, context_lens, B, Hq, Hkv, D,
                             d->block_size, scale, attn, mode);
  else
    orc_attn_decode_paged(q, c->k, c->v, block_table, max_blocks_per_seq,
                          context_lens, B, Hq, Hkv, D, d->block_size, scale,
                          attn, mode);
  layer_tail(d, w, x, attn, y, h_out, B, mode);
  free(pos);
  free(seq);
  free(n1);
  free(q);
  free(k);
  free(v);
  free(attn);
}

/* Float caches [num_blocks][Hkv][BS][D] (k_cache NULL: no cache write). */
void orc_layer_prefill(const orc_dims* d, const orc_weights* w, const float* x,
                       float* y, float* h_out, const int32_t* pos,
                       const int32_t* seq_of_token, const int32_t* cu_seqlens,
                       int B, int T, float* k_cache, float* v_cache,
                       const int32_t* block_table, int max_blocks_per_seq,
                       int mode) {
  const orc_kv c = {k_cache, v_cache, NULL, NULL, NULL, NULL};
  layer_prefill(d, w, x, y, h_out, pos, seq_of_token, cu_seqlens, B, T, &c,
                block_table, max_blocks_per_seq, mode);
}

void orc_layer_decode(const orc_dims* d, const orc_weights* w, const float* x,
                      float* y, float* h_out, const int32_t* context_lens, int B,
                      float* k_cache, float* v_cache, const int32_t* block_table,
                      int max_blocks_per_seq, int mode) {
  const orc_kv c = {k_cache, v_cache, NULL, NULL, NULL, NULL};
  layer_decode(d, w, x, y, h_out, context_lens, B, &c, block_table,
               max_blocks_per_seq, mode);
}

/*
 * A step that brings q_len_b new tokens to every sequence (speculative
 * verification, or a chunk of a prefill over a cached prefix)   [spec]
 * x, y [T][H] packed by cu_q; pos [T] = context_lens[b] - q_len_b + i;
 * seq_of_token [T].  The new tokens' K/V are written to the cache first;
 * attention is orc_attn_paged_qlens over the cache.
 */
void orc_layer_decode_qlens(const orc_dims* d, const orc_weights* w, const float* x,
                            float* y, float* h_out, const int32_t* pos,
                            const int32_t* seq_of_token, const int32_t* cu_q,
                            const int32_t* context_lens, int B, int T,
                            float* k_cache, float* v_cache,
                            const int32_t* block_table, int max_blocks_per_seq,
                            int mode) {
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  float* n1 = (float*)malloc(sizeof(float) * (size_t)T * H);
  float* q = (float*)malloc(sizeof(float) * (size_t)T * Hq * D);
  float* k = (float*)malloc(sizeof(float) * (size_t)T * Hkv * D);
  float* v = (float*)malloc(sizeof(float) * (size_t)T * Hkv * D);
  float* attn = (float*)malloc(sizeof(float) * (size_t)T * Hq * D);
  orc_rmsnorm(x, NULL, NULL, w->ln1, n1, T, H, d->rms_eps, mode);
  orc_qkv_rope(n1, w->wq, w->wk, w->wv, pos, d->rope_theta, q, k, v, T, H, Hq,
               Hkv, D, mode);
  orc_reshape_and_cache(k, v, seq_of_token, pos, block_table, max_blocks_per_seq,
                        k_cache, v_cache, T, Hkv, D, d->block_size);
  orc_attn_paged_qlens(q, k_cache, v_cache, block_table, max_blocks_per_seq, cu_q,
                       context_lens, B, Hq, Hkv, D, d->block_size,
                       1.0 / sqrt((double)D), attn, mode);
  layer_tail(d, w, x, attn, y, h_out, T, mode);
  free(n1);
  free(q);
  free(k);
  free(v);
  free(attn);
}

/* INT8 cache: codes [num_blocks][Hkv][BS][D], scales [num_blocks][Hkv][BS]. */
void orc_layer_prefill_q8(const orc_dims* d, const orc_weights* w, const float* x,
                          float* y, float* h_out, const int32_t* pos,
                          const int32_t* seq_of_token, const int32_t* cu_seqlens,
                          int B, int T, int8_t* k_codes, int8_t* v_codes,
                          float* k_scale, float* v_scale,
                          const int32_t* block_table, int max_blocks_per_seq,
                          int mode) {
  const orc_kv c = {NULL, NULL, k_codes, v_codes, k_scale, v_scale};
  layer_prefill(d, w, x, y, h_out, pos, seq_of_token, cu_seqlens, B, T, &c,
                block_table, max_blocks_per_seq, mode);
}

void orc_layer_decode_q8(const orc_dims* d, const orc_weights* w, const float* x,
                         float* y, float* h_out, const int32_t* context_lens,
                         int B, int8_t* k_codes, int8_t* v_codes, float* k_scale,
                         float* v_scale, const int32_t* block_table,
                         int max_blocks_per_seq, int mode) {
  const orc_kv c = {NULL, NULL, k_codes, v_codes, k_scale, v_scale};
  layer_decode(d, w, x, y, h_out, context_lens, B, &c, block_table,
               max_blocks_per_seq, mode);
}

/* ------------------------------------------------------------------------ */
/* KV-cache size   [kvpage]: bytes = 2 * L * s * b * d * sizeof(dtype)       */
/* ------------------------------------------------------------------------ */

/* d_kv = number of KV heads x head dim (equals hidden for multi-head). */
double orc_kv_cache_bytes(int layers, int64_t seq, int64_t batch, int64_t d_kv,
                          int elem_bytes) {
  return 2.0 * layers * (double)seq * (double)batch * (double)d_kv * elem_bytes;
}
