// capi.hip -- the extern "C" boundary: argument validation, workspace
// planning and carving, and the layer composition (fused and kernel-per-op).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/dl_layer.h"
#include "dl_internal.hpp"

using namespace dl;

namespace {

thread_local std::string g_last_error;

dl_status fail(dl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dl_status fail(dl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dl_status ok() {
  g_last_error.clear();
  return DL_OK;
}

dl_status hip_fail(hipError_t e, const char* where) {
  return fail(DL_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define DL_HIP(call, where)                      \
  do {                                           \
    hipError_t e_ = (call);                      \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// The scaled dot-product's default scale, 1/sqrt(D) (ATB decoder-layer page,
// "operator fusion graph of a decoder layer").
float default_scale(int D) { return 1.0f / sqrtf((float)D); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(dl_dtype dt) { return dt == DL_BF16 ? 2 : 4; }

// ---- shared checks ---------------------------------------------------------
#define CHECK_PTR(p)                                                          \
  do {                                                                        \
    if (!(p)) return fail(DL_ERR_INVALID_ARG, "%s must not be NULL", #p);    \
    if (!aligned16(p)) return fail(DL_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p); \
  } while (0)
#define CHECK_PTR_OPT(p)                                                      \
  do {                                                                        \
    if ((p) && !aligned16(p)) return fail(DL_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p); \
  } while (0)
#define CHECK_IDX(p)                                                          \
  do {                                                                        \
    if (!(p)) return fail(DL_ERR_INVALID_ARG, "%s must not be NULL", #p);    \
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0)                           \
      return fail(DL_ERR_ALIGNMENT, "%s is not 4-byte aligned", #p);         \
  } while (0)

dl_status check_dtype(dl_dtype dt) {
  if (dt != DL_F32 && dt != DL_BF16) return fail(DL_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  return DL_OK;
}

dl_status check_heads(int Hq, int Hkv, int D) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0) return fail(DL_ERR_INVALID_ARG, "heads/head_dim must be positive");
  if (Hq % Hkv) return fail(DL_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  const int g = Hq / Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(DL_ERR_UNSUPPORTED, "Hq/Hkv = %d not in {1,2,4,8}", g);
  if (D != 64 && D != 128) return fail(DL_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", D);
  return DL_OK;
}

dl_status check_hidden(int H) {
  if (H <= 0) return fail(DL_ERR_INVALID_ARG, "hidden must be positive");
  if (H % 32 || H > 8192) return fail(DL_ERR_UNSUPPORTED, "hidden %d must be a multiple of 32 and <= 8192", H);
  return DL_OK;
}

dl_status check_inter(int I) {
  if (I <= 0) return fail(DL_ERR_INVALID_ARG, "intermediate must be positive");
  if (I % 16) return fail(DL_ERR_UNSUPPORTED, "intermediate %d must be a multiple of 16", I);
  return DL_OK;
}

dl_status check_bs(int BS) {
  if (BS != 16 && BS != 32 && BS != 64 && BS != 128)
    return fail(DL_ERR_UNSUPPORTED, "block_size %d not in {16,32,64,128}", BS);
  return DL_OK;
}

#define TRY(expr)                  \
  do {                             \
    dl_status s_ = (expr);         \
    if (s_ != DL_OK) return s_;    \
  } while (0)

// ---- GEMM plans used by each step -----------------------------------------
GemmPlan plan_qkv(int M, int H, int Hq, int Hkv, int D, dl_dtype dt) {
  return plan_gemm(M, (Hq + 2 * Hkv) * D, H, dt == DL_F32, true);
}
GemmPlan plan_lin(int M, int N, int K, dl_dtype dt) { return plan_gemm(M, N, K, dt == DL_F32, false); }
GemmPlan plan_gu(int M, int H, int I, dl_dtype dt) { return plan_gemm(M, 2 * I, H, dt == DL_F32, true); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- layer workspace layout -------------------------------------------------
enum Buf { kN1, kQ, kK, kV, kAttn, kO, kH, kN2, kA, kPart, kDec, kS, kP, kG, kU, kSG, kDd, kNBuf };
static_assert(kN1 == DL_WS_N1 && kQ == DL_WS_Q && kK == DL_WS_K && kV == DL_WS_V &&
                  kAttn == DL_WS_ATTN && kO == DL_WS_O && kH == DL_WS_H && kN2 == DL_WS_N2 &&
                  kA == DL_WS_A && kPart == DL_WS_PARTIAL && kDec == DL_WS_DECODE &&
                  kS == DL_WS_SCORES && kP == DL_WS_PROBS && kG == DL_WS_GATE && kU == DL_WS_UP &&
                  kSG == DL_WS_SILU && kDd == DL_WS_DOWN && kNBuf == DL_WS_COUNT,
              "workspace regions follow the public enum");

struct Layout {
  size_t off[kNBuf];
  size_t size[kNBuf];
  size_t total;
};

size_t part_bytes(const dl_layer_dims* d, int M, dl_mode m) {
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim,
            I = d->intermediate;
  const dl_dtype dt = d->dtype;
  size_t p = 0;
  if (m == DL_FUSED) {
    p = std::max(p, plan_qkv(M, H, Hq, Hkv, D, dt).ws_bytes);
    p = std::max(p, plan_gu(M, H, I, dt).ws_bytes);
  } else {
    p = std::max(p, plan_lin(M, Hq * D, H, dt).ws_bytes);
    p = std::max(p, plan_lin(M, Hkv * D, H, dt).ws_bytes);
    p = std::max(p, plan_lin(M, I, H, dt).ws_bytes);
  }
  p = std::max(p, plan_lin(M, H, Hq * D, dt).ws_bytes);
  p = std::max(p, plan_lin(M, H, I, dt).ws_bytes);
  return p;
}

// is_decode: T = B tokens, S_or_ctx = max context; else S_or_ctx = max_seqlen.
// max_q_len > 0: a step with several new tokens per sequence (S_or_ctx = max
// context), whose attention partials take the decode slot.
Layout layout(const dl_layer_dims* d, int T, int B, int S_or_ctx, bool is_decode, dl_mode m,
              size_t part, int max_q_len = 0) {
  const size_t es = esize(d->dtype);
  const size_t H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim,
               I = d->intermediate;
  Layout L{};
  L.size[kN1] = T * H * es;
  L.size[kQ] = T * Hq * D * es;
  L.size[kK] = T * Hkv * D * es;
  L.size[kV] = T * Hkv * D * es;
  L.size[kAttn] = T * Hq * D * es;
  L.size[kO] = T * H * es;
  L.size[kH] = T * H * 4;
  L.size[kN2] = T * H * es;
  L.size[kA] = T * I * es;
  L.size[kPart] = part;
  L.size[kDec] = is_decode && m == DL_FUSED
                     ? plan_decode(B, (int)Hq, (int)Hkv, (int)D, S_or_ctx, d->block_size).ws_bytes
                     : 0;
  if (max_q_len > 0)
    L.size[kDec] = plan_paged(B, (int)Hq, (int)Hkv, max_q_len, S_or_ctx, d->block_size, (int)D, T)
                       .ws_bytes;
  if (m == DL_UNFUSED) {
    const size_t rows = is_decode ? (size_t)B * Hq : (size_t)B * Hq * S_or_ctx;
    L.size[kS] = rows * S_or_ctx * 4;
    L.size[kP] = rows * S_or_ctx * es;
    L.size[kG] = T * I * es;
    L.size[kU] = T * I * es;
    L.size[kSG] = T * I * es;
    L.size[kDd] = T * H * 4;
  }
  size_t o = 0;
  for (int i = 0; i < kNBuf; ++i) {
    L.off[i] = o;
    o += align256(L.size[i]);
  }
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, const Layout& L, Buf b) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + L.off[b]);
}

dl_status check_dims(const dl_layer_dims* d) {
  if (!d) return fail(DL_ERR_INVALID_ARG, "dims must not be NULL");
  TRY(check_dtype(d->dtype));
  TRY(check_hidden(d->hidden));
  TRY(check_heads(d->n_q_heads, d->n_kv_heads, d->head_dim));
  TRY(check_inter(d->intermediate));
  TRY(check_bs(d->block_size));
  if (!(d->rms_eps >= 0.f)) return fail(DL_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if ((d->n_q_heads * d->head_dim) % 32)
    return fail(DL_ERR_UNSUPPORTED, "Hq*D must be a multiple of 32");
  return DL_OK;
}

dl_status check_weights(const dl_layer_weights* w) {
  if (!w) return fail(DL_ERR_INVALID_ARG, "weights must not be NULL");
  CHECK_PTR(w->ln1_gamma);
  CHECK_PTR(w->w_q);
  CHECK_PTR(w->w_k);
  CHECK_PTR(w->w_v);
  CHECK_PTR(w->w_o);
  CHECK_PTR(w->ln2_gamma);
  CHECK_PTR(w->w_gate);
  CHECK_PTR(w->w_up);
  CHECK_PTR(w->w_down);
  return DL_OK;
}

dl_status check_cache(const dl_kv_cache* c) {
  if (!c) return fail(DL_ERR_INVALID_ARG, "cache must not be NULL");
  CHECK_PTR(c->k_cache);
  CHECK_PTR(c->v_cache);
  if (c->num_blocks <= 0) return fail(DL_ERR_INVALID_ARG, "cache num_blocks must be positive");
  if (c->format != DL_KV_LAYER && c->format != DL_KV_INT8)
    return fail(DL_ERR_INVALID_ARG, "unknown cache format %d", (int)c->format);
  if (c->format == DL_KV_INT8) {
    CHECK_IDX(c->k_scale);
    CHECK_IDX(c->v_scale);
  }
  return DL_OK;
}

bool is_q8(const dl_kv_cache* c) { return c->format == DL_KV_INT8; }

// ---- layer bodies ------------------------------------------------------------
// max_q_len > 0: new tokens appended to cached sequences (cu = cu_q_lens,
// ctx = context lengths, S_or_ctx = max context); attention reads the cache.
template <typename T>
dl_status layer_body(const dl_layer_dims* d, const dl_layer_weights* w, const float* cs,
                     int max_pos, const float* x, float* y, const int32_t* pos, const int32_t* seq,
                     const int32_t* cu, const int32_t* ctx, int B, int Tn, int S_or_ctx,
                     bool is_decode, const dl_kv_cache* cache, const int32_t* bt, int maxblk,
                     dl_mode m, void* ws, const Layout& L, hipStream_t st, int max_q_len = 0) {
  const int H = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim,
            I = d->intermediate, BS = d->block_size;
  const dl_dtype dt = d->dtype;
  const float scale = default_scale(D);
  T* n1 = at<T>(ws, L, kN1);
  T* q = at<T>(ws, L, kQ);
  T* k = at<T>(ws, L, kK);
  T* v = at<T>(ws, L, kV);
  T* attn = at<T>(ws, L, kAttn);
  T* o = at<T>(ws, L, kO);
  float* h = at<float>(ws, L, kH);
  T* n2 = at<T>(ws, L, kN2);
  T* a = at<T>(ws, L, kA);
  void* part = at<void>(ws, L, kPart);
  const T* g1 = static_cast<const T*>(w->ln1_gamma);
  const T* g2 = static_cast<const T*>(w->ln2_gamma);
  const T* wq = static_cast<const T*>(w->w_q);
  const T* wk = static_cast<const T*>(w->w_k);
  const T* wv = static_cast<const T*>(w->w_v);
  const T* wo = static_cast<const T*>(w->w_o);
  const T* wg = static_cast<const T*>(w->w_gate);
  const T* wu = static_cast<const T*>(w->w_up);
  const T* wd = static_cast<const T*>(w->w_down);
  T* kc = static_cast<T*>(cache->k_cache);
  T* vc = static_cast<T*>(cache->v_cache);
  const bool q8 = is_q8(cache);
  int8_t* kq = static_cast<int8_t*>(cache->k_cache);
  int8_t* vq = static_cast<int8_t*>(cache->v_cache);

  DL_HIP((rmsnorm_residual<float, T>(x, nullptr, nullptr, g1, n1, Tn, H, d->rms_eps, st)), "norm1");
  if (q8) {
    // INT8 cache (fused mode only): the projection writes k and v, and the
    // quantising cache write reduces each row to its codes and scale
    DL_HIP(gemm_qkv_rope<T>(n1, wq, wk, wv, pos, cs, max_pos, q, k, v, Tn, H, Hq, Hkv, D,
                            plan_qkv(Tn, H, Hq, Hkv, D, dt), part, st), "qkv_rope");
    DL_HIP(reshape_and_cache_q8<T>(k, v, seq, pos, bt, maxblk, kq, vq, cache->k_scale,
                                   cache->v_scale, Tn, Hkv, D, BS, cache->num_blocks, st),
           "reshape_and_cache_q8");
  } else if (m == DL_FUSED) {
    // the projection's epilogue writes rotated k and v straight into the
    // paged cache (the reshape-and-cache write folded into the QKV step).
    // Decode attention reads them only from there, so k/v are not stored
    // elsewhere (nor for a step with several new tokens per sequence, whose
    // attention also reads the cache); prefill attention reads the
    // contiguous k/v the same epilogue also stores.  The epilogue hands out each output row from LDS
    // in 8-column chunks, so a (token, kv head) cache row leaves as whole
    // 128-byte segments.
    KVSink kv;
    kv.k_cache = kc;
    kv.v_cache = vc;
    kv.seq_of_token = seq;
    kv.block_table = bt;
    kv.max_blocks = maxblk;
    kv.block_size = BS;
    kv.num_blocks = cache->num_blocks;
    const bool kv_bufs = !is_decode && max_q_len == 0;   // only prefill attention reads them
    DL_HIP(gemm_qkv_rope<T>(n1, wq, wk, wv, pos, cs, max_pos, q, kv_bufs ? k : nullptr,
                            kv_bufs ? v : nullptr, Tn, H, Hq, Hkv, D,
                            plan_qkv(Tn, H, Hq, Hkv, D, dt), part, st, kv),
           "qkv_rope_cache");
  } else {
    DL_HIP((gemm_linear<T, T>(n1, wq, q, Tn, Hq * D, H, plan_lin(Tn, Hq * D, H, dt), part, st)), "q");
    DL_HIP((gemm_linear<T, T>(n1, wk, k, Tn, Hkv * D, H, plan_lin(Tn, Hkv * D, H, dt), part, st)), "k");
    DL_HIP((gemm_linear<T, T>(n1, wv, v, Tn, Hkv * D, H, plan_lin(Tn, Hkv * D, H, dt), part, st)), "v");
    DL_HIP(unf_rope<T>(q, pos, cs, max_pos, Tn, Hq, D, st), "rope q");
    DL_HIP(unf_rope<T>(k, pos, cs, max_pos, Tn, Hkv, D, st), "rope k");
    DL_HIP(reshape_and_cache<T>(k, v, seq, pos, bt, maxblk, kc, vc, Tn, Hkv, D, BS,
                                cache->num_blocks, st), "reshape_and_cache");
  }
  if (max_q_len > 0) {
    const PagedPlan pp = plan_paged(B, Hq, Hkv, max_q_len, S_or_ctx, BS, D, Tn);
    DL_HIP(attn_paged_qlens<T>(q, kc, vc, bt, maxblk, cu, ctx, B, Tn, Hq, Hkv, D, BS, S_or_ctx,
                               scale, attn, pp, at<void>(ws, L, kDec), cache->num_blocks, st),
           "attn_paged_qlens");
  } else if (!is_decode) {
    if (m == DL_FUSED) {
      DL_HIP(attn_prefill<T>(q, k, v, cu, B, S_or_ctx, Hq, Hkv, D, scale, attn, st), "attn_prefill");
    } else {
      float* S = at<float>(ws, L, kS);
      T* P = at<T>(ws, L, kP);
      DL_HIP(unf_scores<T>(q, k, cu, B, S_or_ctx, Hq, Hkv, D, scale, S, st), "scores");
      DL_HIP(unf_softmax<T>(S, P, cu, true, B, S_or_ctx, Hq, S_or_ctx, st), "softmax");
      DL_HIP(unf_pv<T>(P, v, cu, B, S_or_ctx, Hq, Hkv, D, attn, st), "pv");
    }
  } else {
    if (m == DL_FUSED && q8) {
      const DecodePlan dp = plan_decode(B, Hq, Hkv, D, S_or_ctx, BS);
      DL_HIP(attn_decode_paged_q8<T>(q, kq, vq, cache->k_scale, cache->v_scale, bt, maxblk, ctx,
                                     B, Hq, Hkv, D, BS, scale, attn, dp, at<void>(ws, L, kDec),
                                     cache->num_blocks, st), "attn_decode_q8");
    } else if (m == DL_FUSED) {
      const DecodePlan dp = plan_decode(B, Hq, Hkv, D, S_or_ctx, BS);
      DL_HIP(attn_decode_paged<T>(q, kc, vc, bt, maxblk, ctx, B, Hq, Hkv, D, BS, scale, attn, dp,
                                  at<void>(ws, L, kDec), cache->num_blocks, st), "attn_decode");
    } else {
      DL_HIP(unf_dec_attn<T>(q, kc, vc, bt, maxblk, ctx, S_or_ctx, B, Hq, Hkv, D, BS, scale,
                             at<float>(ws, L, kS), at<T>(ws, L, kP), attn, cache->num_blocks, st),
             "dec_attn");
    }
  }
  DL_HIP((gemm_linear<T, T>(attn, wo, o, Tn, H, Hq * D, plan_lin(Tn, H, Hq * D, dt), part, st)), "o_proj");
  if (m == DL_FUSED) {
    DL_HIP((rmsnorm_residual<T, T>(o, x, h, g2, n2, Tn, H, d->rms_eps, st)), "norm2");
    DL_HIP(gemm_swiglu<T>(n2, wg, wu, a, Tn, H, I, plan_gu(Tn, H, I, dt), part, st), "gate_up");
    DL_HIP(gemm_linear_resid<T>(a, wd, h, y, Tn, H, I, plan_lin(Tn, H, I, dt), part, st), "down");
  } else {
    T* g = at<T>(ws, L, kG);
    T* u = at<T>(ws, L, kU);
    T* sg = at<T>(ws, L, kSG);
    float* dd = at<float>(ws, L, kDd);
    const int64_t nth = (int64_t)Tn * H, nti = (int64_t)Tn * I;
    DL_HIP(unf_add<T>(x, o, h, nth, st), "add1");
    DL_HIP((rmsnorm_residual<float, T>(h, nullptr, nullptr, g2, n2, Tn, H, d->rms_eps, st)), "norm2");
    DL_HIP((gemm_linear<T, T>(n2, wg, g, Tn, I, H, plan_lin(Tn, I, H, dt), part, st)), "gate");
    DL_HIP((gemm_linear<T, T>(n2, wu, u, Tn, I, H, plan_lin(Tn, I, H, dt), part, st)), "up");
    DL_HIP(unf_silu<T>(g, sg, nti, st), "silu");
    DL_HIP(unf_mul<T>(sg, u, a, nti, st), "mul");
    DL_HIP((gemm_linear<T, float>(a, wd, dd, Tn, H, I, plan_lin(Tn, H, I, dt), part, st)), "down");
    DL_HIP(unf_add<float>(h, dd, y, nth, st), "add2");
  }
  return ok();
}

}  // namespace

// ============================================================================
// extern "C"
// ============================================================================
extern "C" {

const char* dl_status_string(dl_status s) {
  switch (s) {
    case DL_OK: return "DL_OK";
    case DL_ERR_INVALID_ARG: return "DL_ERR_INVALID_ARG";
    case DL_ERR_UNSUPPORTED: return "DL_ERR_UNSUPPORTED";
    case DL_ERR_ALIGNMENT: return "DL_ERR_ALIGNMENT";
    case DL_ERR_WORKSPACE: return "DL_ERR_WORKSPACE";
    case DL_ERR_HIP: return "DL_ERR_HIP";
  }
  return "DL_ERR_UNKNOWN";
}

const char* dl_last_error(void) { return g_last_error.c_str(); }

int32_t dl_abi_version(void) { return 3; }

dl_status dl_rope_table_fill(float* cos_sin, int32_t max_pos, int32_t head_dim, double theta,
                             void* stream) {
  CHECK_PTR(cos_sin);
  if (max_pos < 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (head_dim <= 0 || head_dim % 8) return fail(DL_ERR_UNSUPPORTED, "head_dim must be a positive multiple of 8");
  if (!(theta > 0.0)) return fail(DL_ERR_INVALID_ARG, "theta must be > 0");
  DL_HIP(rope_table_fill(cos_sin, max_pos, head_dim, theta, (hipStream_t)stream), "rope_table");
  return ok();
}

dl_status dl_rmsnorm_residual(const void* x, dl_dtype x_dtype, const float* residual_in,
                              float* residual_out, const void* gamma, void* out, int32_t T,
                              int32_t H, float eps, dl_dtype out_dtype, void* stream) {
  TRY(check_dtype(x_dtype));
  TRY(check_dtype(out_dtype));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  TRY(check_hidden(H));
  if (!(eps >= 0.f)) return fail(DL_ERR_INVALID_ARG, "eps must be >= 0");
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(gamma);
  CHECK_PTR(out);
  CHECK_PTR_OPT(residual_in);
  if (residual_in) CHECK_PTR(residual_out);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (x_dtype == DL_F32 && out_dtype == DL_BF16)
    e = rmsnorm_residual<float, bf16>((const float*)x, residual_in, residual_out, (const bf16*)gamma, (bf16*)out, T, H, eps, st);
  else if (x_dtype == DL_BF16 && out_dtype == DL_BF16)
    e = rmsnorm_residual<bf16, bf16>((const bf16*)x, residual_in, residual_out, (const bf16*)gamma, (bf16*)out, T, H, eps, st);
  else if (x_dtype == DL_F32 && out_dtype == DL_F32)
    e = rmsnorm_residual<float, float>((const float*)x, residual_in, residual_out, (const float*)gamma, (float*)out, T, H, eps, st);
  else
    e = rmsnorm_residual<bf16, float>((const bf16*)x, residual_in, residual_out, (const float*)gamma, (float*)out, T, H, eps, st);
  DL_HIP(e, "rmsnorm");
  return ok();
}

size_t dl_qkv_rope_workspace_size(int32_t T, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                                  dl_dtype dt) {
  if (T <= 0 || H <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
  return plan_qkv(T, H, Hq, Hkv, D, dt).ws_bytes;
}

dl_status dl_qkv_rope(const void* x, const void* w_q, const void* w_k, const void* w_v,
                      const int32_t* positions, const float* cos_sin, int32_t max_pos, void* q,
                      void* k, void* v, int32_t T, int32_t H, int32_t Hq, int32_t Hkv, int32_t D,
                      dl_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  TRY(check_heads(Hq, Hkv, D));
  if (H <= 0 || H % 8) return fail(DL_ERR_UNSUPPORTED, "H must be a positive multiple of 8");
  if (max_pos <= 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be positive");
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w_q);
  CHECK_PTR(w_k);
  CHECK_PTR(w_v);
  CHECK_IDX(positions);
  CHECK_PTR(cos_sin);
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  const GemmPlan pl = plan_qkv(T, H, Hq, Hkv, D, dt);
  if (pl.ws_bytes > ws_bytes || (pl.ws_bytes && !ws))
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR_OPT(ws);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? gemm_qkv_rope<bf16>((const bf16*)x, (const bf16*)w_q, (const bf16*)w_k, (const bf16*)w_v, positions, cos_sin, max_pos, (bf16*)q, (bf16*)k, (bf16*)v, T, H, Hq, Hkv, D, pl, ws, st)
      : gemm_qkv_rope<float>((const float*)x, (const float*)w_q, (const float*)w_k, (const float*)w_v, positions, cos_sin, max_pos, (float*)q, (float*)k, (float*)v, T, H, Hq, Hkv, D, pl, ws, st);
  DL_HIP(e, "qkv_rope");
  return ok();
}

dl_status dl_qkv_rope_cache(const void* x, const void* w_q, const void* w_k, const void* w_v,
                            const int32_t* positions, const float* cos_sin, int32_t max_pos,
                            void* q, void* k, void* v, const int32_t* seq_of_token,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const dl_kv_cache* cache, int32_t T, int32_t H, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t BS, dl_dtype dt, void* ws,
                            size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  TRY(check_heads(Hq, Hkv, D));
  TRY(check_bs(BS));
  if (H <= 0 || H % 8) return fail(DL_ERR_UNSUPPORTED, "H must be a positive multiple of 8");
  if (max_pos <= 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be positive");
  if (max_blocks_per_seq <= 0) return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  TRY(check_cache(cache));
  if (is_q8(cache))
    return fail(DL_ERR_UNSUPPORTED, "the epilogue cache write takes layer-dtype caches; write an "
                                    "INT8 cache with dl_qkv_rope + dl_reshape_and_cache");
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w_q);
  CHECK_PTR(w_k);
  CHECK_PTR(w_v);
  CHECK_IDX(positions);
  CHECK_PTR(cos_sin);
  CHECK_PTR(q);
  if ((k == nullptr) != (v == nullptr)) return fail(DL_ERR_INVALID_ARG, "k and v must both be given or both be NULL");
  if (k) {
    CHECK_PTR(k);
    CHECK_PTR(v);
  }
  if (seq_of_token) CHECK_IDX(seq_of_token);
  CHECK_IDX(block_table);
  const GemmPlan pl = plan_qkv(T, H, Hq, Hkv, D, dt);
  if (pl.ws_bytes > ws_bytes || (pl.ws_bytes && !ws))
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR_OPT(ws);
  KVSink kv;
  kv.k_cache = cache->k_cache;
  kv.v_cache = cache->v_cache;
  kv.seq_of_token = seq_of_token;
  kv.block_table = block_table;
  kv.max_blocks = max_blocks_per_seq;
  kv.block_size = BS;
  kv.num_blocks = cache->num_blocks;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? gemm_qkv_rope<bf16>((const bf16*)x, (const bf16*)w_q, (const bf16*)w_k, (const bf16*)w_v, positions, cos_sin, max_pos, (bf16*)q, (bf16*)k, (bf16*)v, T, H, Hq, Hkv, D, pl, ws, st, kv)
      : gemm_qkv_rope<float>((const float*)x, (const float*)w_q, (const float*)w_k, (const float*)w_v, positions, cos_sin, max_pos, (float*)q, (float*)k, (float*)v, T, H, Hq, Hkv, D, pl, ws, st, kv);
  DL_HIP(e, "qkv_rope_cache");
  return ok();
}

dl_status dl_reshape_and_cache(const void* k, const void* v, const int32_t* seq_of_token,
                               const int32_t* positions, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const dl_kv_cache* cache, int32_t T,
                               int32_t Hkv, int32_t D, int32_t BS, dl_dtype dt, void* stream) {
  TRY(check_dtype(dt));
  if (T < 0 || Hkv <= 0) return fail(DL_ERR_INVALID_ARG, "bad T/Hkv");
  if (D != 64 && D != 128) return fail(DL_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", D);
  TRY(check_bs(BS));
  if (max_blocks_per_seq <= 0) return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  TRY(check_cache(cache));
  if (T == 0) return ok();
  CHECK_PTR(k);
  CHECK_PTR(v);
  if (seq_of_token) CHECK_IDX(seq_of_token);
  CHECK_IDX(positions);
  CHECK_IDX(block_table);
  hipStream_t st = (hipStream_t)stream;
  if (is_q8(cache)) {
    int8_t* kq = static_cast<int8_t*>(cache->k_cache);
    int8_t* vq = static_cast<int8_t*>(cache->v_cache);
    hipError_t e = dt == DL_BF16
        ? reshape_and_cache_q8<bf16>((const bf16*)k, (const bf16*)v, seq_of_token, positions, block_table, max_blocks_per_seq, kq, vq, cache->k_scale, cache->v_scale, T, Hkv, D, BS, cache->num_blocks, st)
        : reshape_and_cache_q8<float>((const float*)k, (const float*)v, seq_of_token, positions, block_table, max_blocks_per_seq, kq, vq, cache->k_scale, cache->v_scale, T, Hkv, D, BS, cache->num_blocks, st);
    DL_HIP(e, "reshape_and_cache_q8");
    return ok();
  }
  hipError_t e = dt == DL_BF16
      ? reshape_and_cache<bf16>((const bf16*)k, (const bf16*)v, seq_of_token, positions, block_table, max_blocks_per_seq, (bf16*)cache->k_cache, (bf16*)cache->v_cache, T, Hkv, D, BS, cache->num_blocks, st)
      : reshape_and_cache<float>((const float*)k, (const float*)v, seq_of_token, positions, block_table, max_blocks_per_seq, (float*)cache->k_cache, (float*)cache->v_cache, T, Hkv, D, BS, cache->num_blocks, st);
  DL_HIP(e, "reshape_and_cache");
  return ok();
}

dl_status dl_attn_prefill(const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t max_seqlen,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, void* out, dl_dtype dt,
                          void* stream) {
  TRY(check_dtype(dt));
  TRY(check_heads(Hq, Hkv, D));
  if (B < 0 || T < 0 || max_seqlen < 0) return fail(DL_ERR_INVALID_ARG, "negative size");
  if (B == 0 || T == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(k);
  CHECK_PTR(v);
  CHECK_PTR(out);
  CHECK_IDX(cu_seqlens);
  if (!(scale > 0.f)) scale = default_scale(D);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? attn_prefill<bf16>((const bf16*)q, (const bf16*)k, (const bf16*)v, cu_seqlens, B, max_seqlen, Hq, Hkv, D, scale, (bf16*)out, st)
      : attn_prefill<float>((const float*)q, (const float*)k, (const float*)v, cu_seqlens, B, max_seqlen, Hq, Hkv, D, scale, (float*)out, st);
  DL_HIP(e, "attn_prefill");
  return ok();
}

size_t dl_attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                     int32_t max_context_len, int32_t BS) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || max_context_len <= 0) return 0;
  return plan_decode(B, Hq, Hkv, D, max_context_len, BS).ws_bytes;
}

}  // extern "C"

namespace {

// ---- fixed device scratch for the entry points that allocate nothing -------
// One array per GPU (each device holds its own copy from the time the library
// is loaded until the process ends).  Host code never uses the array's name as
// an address: the per-device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dl_status scratch_address(void** out) {
  int dev = -1;
  DL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DL_ERR_UNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DL_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DL_OK;
}

dl_status attn_decode_paged_impl(const void* q, const dl_kv_cache* cache,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, float scale,
                                 void* out, dl_dtype dt, void* ws, size_t ws_bytes, bool no_alloc,
                                 void* stream) {
  TRY(check_dtype(dt));
  TRY(check_heads(Hq, Hkv, D));
  TRY(check_bs(BS));
  if (B < 0) return fail(DL_ERR_INVALID_ARG, "B must be >= 0");
  if (max_context_len <= 0) return fail(DL_ERR_INVALID_ARG, "max_context_len must be positive");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * BS < max_context_len)
    return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq * BS must cover max_context_len");
  TRY(check_cache(cache));
  if (B == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(out);
  CHECK_IDX(block_table);
  CHECK_IDX(context_lens);
  const DecodePlan pl = plan_decode(B, Hq, Hkv, D, max_context_len, BS);
  if (no_alloc) {
    if (pl.ws_bytes > kScratchBytes)
      return fail(DL_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch, beyond the fixed %zu-byte device "
                  "scratch of dl_attn_decode_paged_noalloc (use dl_attn_decode_paged with a "
                  "workspace)", pl.ws_bytes, kScratchBytes);
    TRY(scratch_address(&ws));
    ws_bytes = kScratchBytes;
  }
  if (!ws || ws_bytes < pl.ws_bytes)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR(ws);
  if (!(scale > 0.f)) scale = default_scale(D);
  hipStream_t st = (hipStream_t)stream;
  if (is_q8(cache)) {
    const int8_t* kq = static_cast<const int8_t*>(cache->k_cache);
    const int8_t* vq = static_cast<const int8_t*>(cache->v_cache);
    hipError_t e = dt == DL_BF16
        ? attn_decode_paged_q8<bf16>((const bf16*)q, kq, vq, cache->k_scale, cache->v_scale, block_table, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, scale, (bf16*)out, pl, ws, cache->num_blocks, st)
        : attn_decode_paged_q8<float>((const float*)q, kq, vq, cache->k_scale, cache->v_scale, block_table, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, scale, (float*)out, pl, ws, cache->num_blocks, st);
    DL_HIP(e, "attn_decode_paged_q8");
    return ok();
  }
  hipError_t e = dt == DL_BF16
      ? attn_decode_paged<bf16>((const bf16*)q, (const bf16*)cache->k_cache, (const bf16*)cache->v_cache, block_table, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, scale, (bf16*)out, pl, ws, cache->num_blocks, st)
      : attn_decode_paged<float>((const float*)q, (const float*)cache->k_cache, (const float*)cache->v_cache, block_table, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, scale, (float*)out, pl, ws, cache->num_blocks, st);
  DL_HIP(e, "attn_decode_paged");
  return ok();
}

}  // namespace

extern "C" {

dl_status dl_attn_decode_paged(const void* q, const dl_kv_cache* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len, int32_t B,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, float scale,
                               void* out, dl_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  return attn_decode_paged_impl(q, cache, block_table, max_blocks_per_seq, context_lens,
                                max_context_len, B, Hq, Hkv, D, BS, scale, out, dt, ws, ws_bytes,
                                false, stream);
}

dl_status dl_attn_decode_paged_noalloc(const void* q, const dl_kv_cache* cache,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                                       float scale, void* out, dl_dtype dt, void* stream) {
  return attn_decode_paged_impl(q, cache, block_table, max_blocks_per_seq, context_lens,
                                max_context_len, B, Hq, Hkv, D, BS, scale, out, dt, nullptr, 0,
                                true, stream);
}

size_t dl_attn_decode_noalloc_max_scratch(void) { return kScratchBytes; }

size_t dl_attn_paged_qlens_workspace_size(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                                          int32_t D, int32_t max_q_len,
                                          int32_t max_context_len, int32_t BS) {
  if (B <= 0 || Tq <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || max_q_len <= 0 ||
      max_context_len <= 0 || Hq % Hkv)
    return 0;
  return plan_paged(B, Hq, Hkv, max_q_len, max_context_len, BS, D, Tq).ws_bytes;
}

dl_status dl_attn_paged_qlens(const void* q, const dl_kv_cache* cache, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                              const int32_t* context_lens, int32_t B, int32_t Tq,
                              int32_t max_q_len, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t BS, float scale, void* out, dl_dtype dt,
                              void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  TRY(check_heads(Hq, Hkv, D));
  TRY(check_bs(BS));
  if (B < 0 || Tq < 0 || max_q_len < 0) return fail(DL_ERR_INVALID_ARG, "negative size");
  if (max_context_len <= 0) return fail(DL_ERR_INVALID_ARG, "max_context_len must be positive");
  if (max_q_len > max_context_len) return fail(DL_ERR_INVALID_ARG, "max_q_len exceeds max_context_len");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * BS < max_context_len)
    return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq * BS must cover max_context_len");
  TRY(check_cache(cache));
  if (is_q8(cache)) return fail(DL_ERR_UNSUPPORTED, "q_len > 1 paged attention takes layer-dtype caches");
  if (B == 0 || Tq == 0 || max_q_len == 0) return ok();
  CHECK_PTR(q);
  CHECK_PTR(out);
  CHECK_IDX(block_table);
  CHECK_IDX(cu_q_lens);
  CHECK_IDX(context_lens);
  const PagedPlan pl = plan_paged(B, Hq, Hkv, max_q_len, max_context_len, BS, D, Tq);
  if ((int64_t)B * pl.max_qt * pl.max_sp * Hkv > 0x7fffffff)
    return fail(DL_ERR_UNSUPPORTED, "grid too large");
  if (!ws || ws_bytes < pl.ws_bytes)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR(ws);
  if (!(scale > 0.f)) scale = default_scale(D);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? attn_paged_qlens<bf16>((const bf16*)q, (const bf16*)cache->k_cache, (const bf16*)cache->v_cache, block_table, max_blocks_per_seq, cu_q_lens, context_lens, B, Tq, Hq, Hkv, D, BS, max_context_len, scale, (bf16*)out, pl, ws, cache->num_blocks, st)
      : attn_paged_qlens<float>((const float*)q, (const float*)cache->k_cache, (const float*)cache->v_cache, block_table, max_blocks_per_seq, cu_q_lens, context_lens, B, Tq, Hq, Hkv, D, BS, max_context_len, scale, (float*)out, pl, ws, cache->num_blocks, st);
  DL_HIP(e, "attn_paged_qlens");
  return ok();
}

size_t dl_linear_workspace_size(int32_t M, int32_t N, int32_t K, dl_dtype dt) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return plan_lin(M, N, K, dt).ws_bytes;
}

dl_status dl_linear(const void* x, const void* w, void* out, int32_t M, int32_t N, int32_t K,
                    dl_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  if (M < 0 || N <= 0 || K <= 0) return fail(DL_ERR_INVALID_ARG, "bad M/N/K");
  if (N % 16 || K % 8) return fail(DL_ERR_UNSUPPORTED, "N must be a multiple of 16 and K of 8");
  if (M == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w);
  CHECK_PTR(out);
  const GemmPlan pl = plan_lin(M, N, K, dt);
  if (pl.ws_bytes > ws_bytes || (pl.ws_bytes && !ws))
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR_OPT(ws);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? gemm_linear<bf16, bf16>((const bf16*)x, (const bf16*)w, (bf16*)out, M, N, K, pl, ws, st)
      : gemm_linear<float, float>((const float*)x, (const float*)w, (float*)out, M, N, K, pl, ws, st);
  DL_HIP(e, "linear");
  return ok();
}

size_t dl_gate_up_silu_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0) return 0;
  return plan_gu(T, H, I, dt).ws_bytes;
}

dl_status dl_gate_up_silu(const void* x, const void* w_gate, const void* w_up, void* a, int32_t T,
                          int32_t H, int32_t I, dl_dtype dt, void* ws, size_t ws_bytes,
                          void* stream) {
  TRY(check_dtype(dt));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  if (H <= 0 || H % 8) return fail(DL_ERR_UNSUPPORTED, "H must be a positive multiple of 8");
  TRY(check_inter(I));
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w_gate);
  CHECK_PTR(w_up);
  CHECK_PTR(a);
  const GemmPlan pl = plan_gu(T, H, I, dt);
  if (pl.ws_bytes > ws_bytes || (pl.ws_bytes && !ws))
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR_OPT(ws);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = dt == DL_BF16
      ? gemm_swiglu<bf16>((const bf16*)x, (const bf16*)w_gate, (const bf16*)w_up, (bf16*)a, T, H, I, pl, ws, st)
      : gemm_swiglu<float>((const float*)x, (const float*)w_gate, (const float*)w_up, (float*)a, T, H, I, pl, ws, st);
  DL_HIP(e, "gate_up_silu");
  return ok();
}

size_t dl_down_residual_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0) return 0;
  return plan_lin(T, H, I, dt).ws_bytes;
}

dl_status dl_down_residual(const void* a, const void* w_down, const float* residual, float* out,
                           int32_t T, int32_t H, int32_t I, dl_dtype dt, void* ws,
                           size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  TRY(check_hidden(H));
  TRY(check_inter(I));
  if (I % 8) return fail(DL_ERR_UNSUPPORTED, "I must be a multiple of 8");
  if (T == 0) return ok();
  CHECK_PTR(a);
  CHECK_PTR(w_down);
  CHECK_PTR_OPT(residual);
  CHECK_PTR(out);
  const GemmPlan pl = plan_lin(T, H, I, dt);
  if (pl.ws_bytes > ws_bytes || (pl.ws_bytes && !ws))
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, pl.ws_bytes);
  CHECK_PTR_OPT(ws);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (residual) {
    e = dt == DL_BF16
        ? gemm_linear_resid<bf16>((const bf16*)a, (const bf16*)w_down, residual, out, T, H, I, pl, ws, st)
        : gemm_linear_resid<float>((const float*)a, (const float*)w_down, residual, out, T, H, I, pl, ws, st);
  } else {
    e = dt == DL_BF16
        ? gemm_linear<bf16, float>((const bf16*)a, (const bf16*)w_down, out, T, H, I, pl, ws, st)
        : gemm_linear<float, float>((const float*)a, (const float*)w_down, out, T, H, I, pl, ws, st);
  }
  DL_HIP(e, "down_residual");
  return ok();
}

size_t dl_ffn_workspace_size(int32_t T, int32_t H, int32_t I, dl_dtype dt) {
  if (T <= 0 || H <= 0 || I <= 0) return 0;
  const size_t a = align256((size_t)T * I * esize(dt));
  return a + std::max(plan_gu(T, H, I, dt).ws_bytes, plan_lin(T, H, I, dt).ws_bytes);
}

dl_status dl_ffn_swiglu(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                        const float* residual, float* out, int32_t T, int32_t H, int32_t I,
                        dl_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dtype(dt));
  if (T < 0) return fail(DL_ERR_INVALID_ARG, "T must be >= 0");
  TRY(check_hidden(H));
  TRY(check_inter(I));
  if (T == 0) return ok();
  CHECK_PTR(x);
  CHECK_PTR(w_gate);
  CHECK_PTR(w_up);
  CHECK_PTR(w_down);
  CHECK_PTR_OPT(residual);
  CHECK_PTR(out);
  const size_t need = dl_ffn_workspace_size(T, H, I, dt);
  if (!ws || ws_bytes < need)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, need);
  CHECK_PTR(ws);
  void* a = ws;
  void* part = static_cast<char*>(ws) + align256((size_t)T * I * esize(dt));
  hipStream_t st = (hipStream_t)stream;
  if (dt == DL_BF16) {
    DL_HIP(gemm_swiglu<bf16>((const bf16*)x, (const bf16*)w_gate, (const bf16*)w_up, (bf16*)a, T, H, I, plan_gu(T, H, I, dt), part, st), "gate_up");
    DL_HIP((residual ? gemm_linear_resid<bf16>((const bf16*)a, (const bf16*)w_down, residual, out, T, H, I, plan_lin(T, H, I, dt), part, st)
                     : gemm_linear<bf16, float>((const bf16*)a, (const bf16*)w_down, out, T, H, I, plan_lin(T, H, I, dt), part, st)), "down");
  } else {
    DL_HIP(gemm_swiglu<float>((const float*)x, (const float*)w_gate, (const float*)w_up, (float*)a, T, H, I, plan_gu(T, H, I, dt), part, st), "gate_up");
    DL_HIP((residual ? gemm_linear_resid<float>((const float*)a, (const float*)w_down, residual, out, T, H, I, plan_lin(T, H, I, dt), part, st)
                     : gemm_linear<float, float>((const float*)a, (const float*)w_down, out, T, H, I, plan_lin(T, H, I, dt), part, st)), "down");
  }
  return ok();
}

size_t dl_layer_workspace_size(const dl_layer_dims* d, int32_t max_tokens, int32_t max_batch,
                               int32_t max_seqlen, int32_t max_context_len, dl_mode m) {
  if (check_dims(d) != DL_OK || max_tokens < 0 || max_batch < 0) return 0;
  if (m != DL_FUSED && m != DL_UNFUSED) return 0;
  // split-K partial needs are not monotonic in M: take the max over every M
  // up to 512 and the largest sizes.
  size_t part = 0;
  const int mt = std::max(max_tokens, max_batch);
  for (int M = 1; M <= std::min(mt, 512); ++M) part = std::max(part, part_bytes(d, M, m));
  part = std::max(part, part_bytes(d, std::max(mt, 1), m));
  size_t need = 0;
  if (max_tokens > 0 && max_batch > 0)
    need = std::max(need, layout(d, max_tokens, max_batch, std::max(max_seqlen, 1), false, m, part).total);
  if (max_batch > 0 && max_context_len > 0)
    need = std::max(need, layout(d, max_batch, max_batch, max_context_len, true, m, part).total);
  return need;
}

dl_status dl_layer_prefill(const dl_layer_dims* d, const dl_layer_weights* w,
                           const float* cos_sin, int32_t max_pos, const float* hidden_in,
                           float* hidden_out, const int32_t* positions,
                           const int32_t* seq_of_token, const int32_t* cu_seqlens, int32_t B,
                           int32_t T, int32_t max_seqlen, const dl_kv_cache* cache,
                           const int32_t* block_table, int32_t max_blocks_per_seq, dl_mode m,
                           void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  TRY(check_weights(w));
  TRY(check_cache(cache));
  if (m != DL_FUSED && m != DL_UNFUSED) return fail(DL_ERR_INVALID_ARG, "unknown mode %d", (int)m);
  if (is_q8(cache) && m != DL_FUSED)
    return fail(DL_ERR_UNSUPPORTED, "INT8 caches run in DL_FUSED mode only");
  if (B < 0 || T < 0 || max_seqlen < 0) return fail(DL_ERR_INVALID_ARG, "negative size");
  if (max_pos <= 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be positive");
  if (max_blocks_per_seq <= 0) return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (T == 0 || B == 0) return ok();
  if (max_seqlen <= 0 || max_seqlen > T) return fail(DL_ERR_INVALID_ARG, "max_seqlen must be in [1, T]");
  CHECK_PTR(cos_sin);
  CHECK_PTR(hidden_in);
  CHECK_PTR(hidden_out);
  if (hidden_in == hidden_out) return fail(DL_ERR_INVALID_ARG, "hidden_out must not alias hidden_in");
  CHECK_IDX(positions);
  CHECK_IDX(seq_of_token);
  CHECK_IDX(cu_seqlens);
  CHECK_IDX(block_table);
  const size_t part = part_bytes(d, T, m);
  const Layout L = layout(d, T, B, max_seqlen, false, m, part);
  if (!ws || ws_bytes < L.total)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, L.total);
  CHECK_PTR(ws);
  hipStream_t st = (hipStream_t)stream;
  if (d->dtype == DL_BF16)
    return layer_body<bf16>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, seq_of_token,
                            cu_seqlens, nullptr, B, T, max_seqlen, false, cache, block_table,
                            max_blocks_per_seq, m, ws, L, st);
  return layer_body<float>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, seq_of_token,
                           cu_seqlens, nullptr, B, T, max_seqlen, false, cache, block_table,
                           max_blocks_per_seq, m, ws, L, st);
}

size_t dl_layer_decode_qlens_workspace_size(const dl_layer_dims* d, int32_t max_tokens,
                                            int32_t max_batch, int32_t max_q_len,
                                            int32_t max_context_len) {
  if (check_dims(d) != DL_OK || max_tokens <= 0 || max_batch <= 0 || max_q_len <= 0 ||
      max_context_len <= 0)
    return 0;
  size_t part = 0;
  for (int M = 1; M <= std::min(max_tokens, 512); ++M)
    part = std::max(part, part_bytes(d, M, DL_FUSED));
  part = std::max(part, part_bytes(d, max_tokens, DL_FUSED));
  return layout(d, max_tokens, max_batch, max_context_len, false, DL_FUSED, part, max_q_len).total;
}

dl_status dl_layer_decode_qlens(const dl_layer_dims* d, const dl_layer_weights* w,
                                const float* cos_sin, int32_t max_pos, const float* hidden_in,
                                float* hidden_out, const int32_t* positions,
                                const int32_t* seq_of_token, const int32_t* cu_q_lens,
                                const int32_t* context_lens, int32_t B, int32_t T,
                                int32_t max_q_len, int32_t max_context_len,
                                const dl_kv_cache* cache, const int32_t* block_table,
                                int32_t max_blocks_per_seq, dl_mode m, void* ws, size_t ws_bytes,
                                void* stream) {
  TRY(check_dims(d));
  TRY(check_weights(w));
  TRY(check_cache(cache));
  if (m != DL_FUSED && m != DL_UNFUSED) return fail(DL_ERR_INVALID_ARG, "unknown mode %d", (int)m);
  if (m != DL_FUSED) return fail(DL_ERR_UNSUPPORTED, "q_len > 1 steps run in DL_FUSED mode only");
  if (is_q8(cache)) return fail(DL_ERR_UNSUPPORTED, "q_len > 1 steps take layer-dtype caches");
  if (B < 0 || T < 0 || max_q_len < 0) return fail(DL_ERR_INVALID_ARG, "negative size");
  if (max_pos <= 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be positive");
  if (max_context_len <= 0) return fail(DL_ERR_INVALID_ARG, "max_context_len must be positive");
  if (max_q_len > max_context_len) return fail(DL_ERR_INVALID_ARG, "max_q_len exceeds max_context_len");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * d->block_size < max_context_len)
    return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq * BS must cover max_context_len");
  if (T == 0 || B == 0 || max_q_len == 0) return ok();
  CHECK_PTR(cos_sin);
  CHECK_PTR(hidden_in);
  CHECK_PTR(hidden_out);
  if (hidden_in == hidden_out) return fail(DL_ERR_INVALID_ARG, "hidden_out must not alias hidden_in");
  CHECK_IDX(positions);
  CHECK_IDX(seq_of_token);
  CHECK_IDX(cu_q_lens);
  CHECK_IDX(context_lens);
  CHECK_IDX(block_table);
  const PagedPlan pp = plan_paged(B, d->n_q_heads, d->n_kv_heads, max_q_len, max_context_len,
                                  d->block_size, d->head_dim, T);
  if ((int64_t)B * pp.max_qt * pp.max_sp * d->n_kv_heads > 0x7fffffff)
    return fail(DL_ERR_UNSUPPORTED, "grid too large");
  const size_t part = part_bytes(d, T, m);
  const Layout L = layout(d, T, B, max_context_len, false, m, part, max_q_len);
  if (!ws || ws_bytes < L.total)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, L.total);
  CHECK_PTR(ws);
  hipStream_t st = (hipStream_t)stream;
  if (d->dtype == DL_BF16)
    return layer_body<bf16>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, seq_of_token,
                            cu_q_lens, context_lens, B, T, max_context_len, false, cache,
                            block_table, max_blocks_per_seq, m, ws, L, st, max_q_len);
  return layer_body<float>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, seq_of_token,
                           cu_q_lens, context_lens, B, T, max_context_len, false, cache,
                           block_table, max_blocks_per_seq, m, ws, L, st, max_q_len);
}

dl_status dl_layer_decode(const dl_layer_dims* d, const dl_layer_weights* w,
                          const float* cos_sin, int32_t max_pos, const float* hidden_in,
                          float* hidden_out, const int32_t* positions,
                          const int32_t* context_lens, int32_t max_context_len, int32_t B,
                          const dl_kv_cache* cache, const int32_t* block_table,
                          int32_t max_blocks_per_seq, dl_mode m, void* ws, size_t ws_bytes,
                          void* stream) {
  TRY(check_dims(d));
  TRY(check_weights(w));
  TRY(check_cache(cache));
  if (m != DL_FUSED && m != DL_UNFUSED) return fail(DL_ERR_INVALID_ARG, "unknown mode %d", (int)m);
  if (is_q8(cache) && m != DL_FUSED)
    return fail(DL_ERR_UNSUPPORTED, "INT8 caches run in DL_FUSED mode only");
  if (B < 0) return fail(DL_ERR_INVALID_ARG, "B must be >= 0");
  if (max_pos <= 0) return fail(DL_ERR_INVALID_ARG, "max_pos must be positive");
  if (max_context_len <= 0) return fail(DL_ERR_INVALID_ARG, "max_context_len must be positive");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * d->block_size < max_context_len)
    return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq * BS must cover max_context_len");
  if (B == 0) return ok();
  CHECK_PTR(cos_sin);
  CHECK_PTR(hidden_in);
  CHECK_PTR(hidden_out);
  if (hidden_in == hidden_out) return fail(DL_ERR_INVALID_ARG, "hidden_out must not alias hidden_in");
  CHECK_IDX(positions);
  CHECK_IDX(context_lens);
  CHECK_IDX(block_table);
  const size_t part = part_bytes(d, B, m);
  const Layout L = layout(d, B, B, max_context_len, true, m, part);
  if (!ws || ws_bytes < L.total)
    return fail(DL_ERR_WORKSPACE, "workspace %zu < required %zu", ws_bytes, L.total);
  CHECK_PTR(ws);
  hipStream_t st = (hipStream_t)stream;
  if (d->dtype == DL_BF16)
    return layer_body<bf16>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, nullptr, nullptr,
                            context_lens, B, B, max_context_len, true, cache, block_table,
                            max_blocks_per_seq, m, ws, L, st);
  return layer_body<float>(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions, nullptr, nullptr,
                           context_lens, B, B, max_context_len, true, cache, block_table,
                           max_blocks_per_seq, m, ws, L, st);
}

dl_status dl_check_indices(const int32_t* block_table, int32_t B, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t BS, const int32_t* positions,
                           const int32_t* seq_of_token, int32_t T, const int32_t* context_lens,
                           int32_t max_context_len, const int32_t* cu_seqlens,
                           int32_t max_seqlen, int32_t* error_word, void* stream) {
  if (!error_word) return fail(DL_ERR_INVALID_ARG, "error_word must not be NULL");
  if ((reinterpret_cast<uintptr_t>(error_word) & 3u) != 0)
    return fail(DL_ERR_ALIGNMENT, "error_word is not 4-byte aligned");
  if (B < 0 || T < 0) return fail(DL_ERR_INVALID_ARG, "negative size");
  if (block_table || positions) {
    TRY(check_bs(BS));
    if (max_blocks_per_seq <= 0) return fail(DL_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  }
  if (block_table && num_blocks <= 0) return fail(DL_ERR_INVALID_ARG, "num_blocks must be positive");
  if (context_lens && max_context_len <= 0)
    return fail(DL_ERR_INVALID_ARG, "max_context_len must be positive");
  if (cu_seqlens && max_seqlen < 0) return fail(DL_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  if (block_table) CHECK_IDX(block_table);
  if (positions) CHECK_IDX(positions);
  if (seq_of_token) CHECK_IDX(seq_of_token);
  if (context_lens) CHECK_IDX(context_lens);
  if (cu_seqlens) CHECK_IDX(cu_seqlens);
  // without positions there are no per-token checks except the sequence map
  const int Tt = (positions || seq_of_token) ? T : 0;
  DL_HIP(check_indices(block_table, B, max_blocks_per_seq, num_blocks, BS, positions,
                       seq_of_token, Tt, context_lens, max_context_len, cu_seqlens, max_seqlen,
                       error_word, (hipStream_t)stream),
         "check_indices");
  return ok();
}

dl_status dl_layer_workspace_regions(const dl_layer_dims* d, int32_t T, int32_t B,
                                     int32_t max_seqlen_or_context, int32_t is_decode, dl_mode m,
                                     size_t* offsets, size_t* sizes) {
  TRY(check_dims(d));
  if (m != DL_FUSED && m != DL_UNFUSED) return fail(DL_ERR_INVALID_ARG, "unknown mode %d", (int)m);
  if (!offsets || !sizes) return fail(DL_ERR_INVALID_ARG, "offsets and sizes must not be NULL");
  if (T <= 0 || B <= 0 || max_seqlen_or_context <= 0)
    return fail(DL_ERR_INVALID_ARG, "T, B and the length bound must be positive");
  if (is_decode && T != B) return fail(DL_ERR_INVALID_ARG, "a decode layout has T == B");
  if (!is_decode && max_seqlen_or_context > T)
    return fail(DL_ERR_INVALID_ARG, "max_seqlen must be in [1, T]");
  const Layout L = layout(d, T, B, max_seqlen_or_context, is_decode != 0, m,
                          part_bytes(d, T, m));
  for (int i = 0; i < kNBuf; ++i) {
    offsets[i] = L.off[i];
    sizes[i] = L.size[i];
  }
  return ok();
}

struct dl_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

dl_status dl_layer_decode_graph_create(const dl_layer_dims* d, const dl_layer_weights* w,
                                       const float* cos_sin, int32_t max_pos,
                                       const float* hidden_in, float* hidden_out,
                                       const int32_t* positions, const int32_t* context_lens,
                                       int32_t max_context_len, int32_t B,
                                       const dl_kv_cache* cache, const int32_t* block_table,
                                       int32_t max_blocks_per_seq, void* ws, size_t ws_bytes,
                                       void* stream, dl_graph* graph) {
  if (!graph) return fail(DL_ERR_INVALID_ARG, "graph must not be NULL");
  if (!stream) return fail(DL_ERR_INVALID_ARG, "capture needs a stream other than the default (NULL) one");
  hipStream_t st = (hipStream_t)stream;
  DL_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal), "begin capture");
  const dl_status s = dl_layer_decode(d, w, cos_sin, max_pos, hidden_in, hidden_out, positions,
                                      context_lens, max_context_len, B, cache, block_table,
                                      max_blocks_per_seq, DL_FUSED, ws, ws_bytes, stream);
  const std::string why = g_last_error;
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(st, &g);
  if (s != DL_OK) {
    if (e == hipSuccess && g) hipGraphDestroy(g);
    g_last_error = why;
    return s;
  }
  if (e != hipSuccess) return hip_fail(e, "end capture");
  hipGraphExec_t x = nullptr;
  const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    hipGraphDestroy(g);
    return hip_fail(ei, "graph instantiate");
  }
  *graph = new dl_graph_s{g, x};
  return ok();
}

dl_status dl_graph_launch(dl_graph graph, void* stream) {
  if (!graph) return fail(DL_ERR_INVALID_ARG, "graph must not be NULL");
  DL_HIP(hipGraphLaunch(graph->exec, (hipStream_t)stream), "graph launch");
  return ok();
}

dl_status dl_graph_destroy(dl_graph graph) {
  if (!graph) return ok();
  const hipError_t e1 = hipGraphExecDestroy(graph->exec);
  const hipError_t e2 = hipGraphDestroy(graph->graph);
  delete graph;
  if (e1 != hipSuccess) return hip_fail(e1, "graph exec destroy");
  if (e2 != hipSuccess) return hip_fail(e2, "graph destroy");
  return ok();
}

}  // extern "C"
