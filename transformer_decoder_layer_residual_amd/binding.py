"""ctypes binding over libdl_layer.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/dl_layer.h).  Tensors are torch CUDA (HIP) tensors; their device
pointers, sizes and the current stream are passed through unchanged, and all
work happens in the HIP kernels behind the C ABI.  Workspaces are allocated
with torch when the caller does not pass one.  There is no fallback: if the
library is missing or the device is not a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdl_layer.so")

DL_OK = 0
DL_F32, DL_BF16 = 0, 1
DL_FUSED, DL_UNFUSED = 0, 1
DL_KV_LAYER, DL_KV_INT8 = 0, 1
ABI_VERSION = 3

_c_int = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class DLError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class LayerDims(ctypes.Structure):
    _fields_ = [("hidden", _c_int), ("n_q_heads", _c_int), ("n_kv_heads", _c_int),
                ("head_dim", _c_int), ("intermediate", _c_int), ("block_size", _c_int),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("ln1_gamma", "w_q", "w_k", "w_v", "w_o", "ln2_gamma",
                                   "w_gate", "w_up", "w_down")]


class KVCache(ctypes.Structure):
    _fields_ = [("k_cache", _vp), ("v_cache", _vp), ("num_blocks", _c_int),
                ("format", ctypes.c_int), ("k_scale", _vp), ("v_scale", _vp)]


# (name, restype, argtypes)
_SIGS = [
    ("dl_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("dl_last_error", ctypes.c_char_p, []),
    ("dl_abi_version", _c_int, []),
    ("dl_rope_table_fill", ctypes.c_int, [_vp, _c_int, _c_int, ctypes.c_double, _vp]),
    ("dl_rmsnorm_residual", ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                           ctypes.c_float, ctypes.c_int, _vp]),
    ("dl_qkv_rope_workspace_size", _sz, [_c_int] * 5 + [ctypes.c_int]),
    ("dl_qkv_rope", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, ctypes.c_int, _vp, _sz, _vp]),
    ("dl_qkv_rope_cache", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
                                         _vp, _c_int, ctypes.POINTER(KVCache), _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, ctypes.c_int, _vp, _sz,
                                         _vp]),
    ("dl_reshape_and_cache", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_int,
                                            ctypes.POINTER(KVCache), _c_int, _c_int, _c_int,
                                            _c_int, ctypes.c_int, _vp]),
    ("dl_attn_prefill", ctypes.c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, ctypes.c_float, _vp, ctypes.c_int, _vp]),
    ("dl_attn_decode_workspace_size", _sz, [_c_int] * 6),
    ("dl_attn_decode_paged", ctypes.c_int, [_vp, ctypes.POINTER(KVCache), _vp, _c_int, _vp,
                                            _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            ctypes.c_float, _vp, ctypes.c_int, _vp, _sz, _vp]),
    ("dl_attn_decode_paged_noalloc", ctypes.c_int, [_vp, ctypes.POINTER(KVCache), _vp, _c_int,
                                                    _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                    _c_int, ctypes.c_float, _vp, ctypes.c_int,
                                                    _vp]),
    ("dl_attn_decode_noalloc_max_scratch", _sz, []),
    ("dl_attn_paged_qlens_workspace_size", _sz, [_c_int] * 8),
    ("dl_attn_paged_qlens", ctypes.c_int, [_vp, ctypes.POINTER(KVCache), _vp, _c_int, _vp, _vp,
                                           _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                           _c_int, _c_int, ctypes.c_float, _vp, ctypes.c_int,
                                           _vp, _sz, _vp]),
    ("dl_linear_workspace_size", _sz, [_c_int, _c_int, _c_int, ctypes.c_int]),
    ("dl_linear", ctypes.c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, ctypes.c_int, _vp, _sz,
                                 _vp]),
    ("dl_ffn_workspace_size", _sz, [_c_int, _c_int, _c_int, ctypes.c_int]),
    ("dl_ffn_swiglu", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                     ctypes.c_int, _vp, _sz, _vp]),
    ("dl_gate_up_silu_workspace_size", _sz, [_c_int, _c_int, _c_int, ctypes.c_int]),
    ("dl_gate_up_silu", ctypes.c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, ctypes.c_int,
                                       _vp, _sz, _vp]),
    ("dl_down_residual_workspace_size", _sz, [_c_int, _c_int, _c_int, ctypes.c_int]),
    ("dl_down_residual", ctypes.c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, ctypes.c_int,
                                        _vp, _sz, _vp]),
    ("dl_layer_workspace_size", _sz, [ctypes.POINTER(LayerDims), _c_int, _c_int, _c_int, _c_int,
                                      ctypes.c_int]),
    ("dl_layer_prefill", ctypes.c_int, [ctypes.POINTER(LayerDims), ctypes.POINTER(LayerWeights),
                                        _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                        _c_int, ctypes.POINTER(KVCache), _vp, _c_int,
                                        ctypes.c_int, _vp, _sz, _vp]),
    ("dl_layer_decode", ctypes.c_int, [ctypes.POINTER(LayerDims), ctypes.POINTER(LayerWeights),
                                       _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                       ctypes.POINTER(KVCache), _vp, _c_int, ctypes.c_int, _vp,
                                       _sz, _vp]),
    ("dl_layer_decode_graph_create", ctypes.c_int,
     [ctypes.POINTER(LayerDims), ctypes.POINTER(LayerWeights), _vp, _c_int, _vp, _vp, _vp, _vp,
      _c_int, _c_int, ctypes.POINTER(KVCache), _vp, _c_int, _vp, _sz, _vp,
      ctypes.POINTER(_vp)]),
    ("dl_graph_launch", ctypes.c_int, [_vp, _vp]),
    ("dl_graph_destroy", ctypes.c_int, [_vp]),
    ("dl_check_indices", ctypes.c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int,
                                        _vp, _c_int, _vp, _c_int, _vp, _vp]),
    ("dl_layer_workspace_regions", ctypes.c_int, [ctypes.POINTER(LayerDims), _c_int, _c_int,
                                                  _c_int, _c_int, ctypes.c_int,
                                                  ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    ("dl_layer_decode_qlens_workspace_size", _sz, [ctypes.POINTER(LayerDims), _c_int, _c_int,
                                                   _c_int, _c_int]),
    ("dl_layer_decode_qlens", ctypes.c_int, [ctypes.POINTER(LayerDims),
                                             ctypes.POINTER(LayerWeights), _vp, _c_int, _vp, _vp,
                                             _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                             ctypes.POINTER(KVCache), _vp, _c_int, ctypes.c_int,
                                             _vp, _sz, _vp]),
]

EXPORTED = tuple(n for n, _, _ in _SIGS)

_lock = threading.Lock()
_lib = None


def lib():
    """Load libdl_layer.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "transformer_decoder_layer_residual_amd.build.build()")
            L = ctypes.CDLL(LIB_PATH)
            for name, res, args in _SIGS:
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _check(status: int):
    if status != DL_OK:
        L = lib()
        raise DLError(status, L.dl_status_string(status).decode(),
                      L.dl_last_error().decode())


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DL_BF16
    if dt == torch.float32:
        return DL_F32
    raise TypeError(f"unsupported dtype {dt}")


def _ws(nbytes: int, ws, device):
    if nbytes == 0:
        return ws, (0 if ws is None else ws.numel() * ws.element_size())
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _cache(k_cache, v_cache, k_scale=None, v_scale=None) -> KVCache:
    """int8 cache tensors describe a DL_KV_INT8 cache (codes) and need the
    [num_blocks, Hkv, BS] float32 row scales; any other dtype is the layer
    dtype."""
    if k_cache.dtype == torch.int8:
        if k_scale is None or v_scale is None:
            raise ValueError("an int8 KV cache needs k_scale and v_scale")
        return KVCache(_p(k_cache), _p(v_cache), int(k_cache.shape[0]), DL_KV_INT8, _p(k_scale),
                       _p(v_scale))
    return KVCache(_p(k_cache), _p(v_cache), int(k_cache.shape[0]), DL_KV_LAYER, None, None)


# ---------------------------------------------------------------------------
# step entry points
# ---------------------------------------------------------------------------

DL_CHECK_BIT_SEQ, DL_CHECK_BIT_POSITION, DL_CHECK_BIT_BLOCK = 1, 2, 4
DL_CHECK_BIT_CONTEXT, DL_CHECK_BIT_CU = 8, 16
WS_REGIONS = ("n1", "q", "k", "v", "attn", "o", "h", "n2", "a", "partial", "decode", "scores",
              "probs", "gate", "up", "silu", "down")


def dl_check_indices(error_word, block_table=None, num_blocks=0, block_size=0, positions=None,
                     seq_of_token=None, context_lens=None, max_context_len=0, cu_seqlens=None,
                     max_seqlen=0, B=None, T=None):
    """Enqueue the index validation; error_word is a 1-element int32 device
    tensor that receives the OR of the violated DL_CHECK_BIT_* bits."""
    if B is None:
        B = (block_table.shape[0] if block_table is not None else
             context_lens.shape[0] if context_lens is not None else
             cu_seqlens.shape[0] - 1 if cu_seqlens is not None else 0)
    if T is None:
        T = (positions.shape[0] if positions is not None else
             seq_of_token.shape[0] if seq_of_token is not None else 0)
    mb = block_table.shape[1] if block_table is not None else 0
    _check(lib().dl_check_indices(_p(block_table), B, mb, num_blocks, block_size, _p(positions),
                                  _p(seq_of_token), T, _p(context_lens), max_context_len,
                                  _p(cu_seqlens), max_seqlen, _p(error_word), _stream()))


def dl_layer_workspace_regions(dims, T: int, B: int, max_seqlen_or_context: int, is_decode: bool,
                               mode=DL_FUSED):
    """{region name: (byte offset, byte size)} of the layer workspace."""
    off = (_sz * len(WS_REGIONS))()
    size = (_sz * len(WS_REGIONS))()
    _check(lib().dl_layer_workspace_regions(ctypes.byref(dims), T, B, max_seqlen_or_context,
                                            int(bool(is_decode)), mode, off, size))
    return {n: (int(off[i]), int(size[i])) for i, n in enumerate(WS_REGIONS)}


def dl_rope_table_fill(cos_sin, max_pos: int, head_dim: int, theta: float):
    _check(lib().dl_rope_table_fill(_p(cos_sin), max_pos, head_dim, theta, _stream()))


def dl_rmsnorm_residual(x, gamma, out, eps: float, residual_in=None, residual_out=None):
    T, H = (x.shape[0], x.shape[1]) if x.dim() == 2 else (0, x.shape[-1])
    _check(lib().dl_rmsnorm_residual(_p(x), dtype_code(x.dtype), _p(residual_in), _p(residual_out),
                                     _p(gamma), _p(out), T, H, eps, dtype_code(out.dtype),
                                     _stream()))


def dl_qkv_rope(x, w_q, w_k, w_v, positions, cos_sin, q, k, v, ws=None):
    T, H = x.shape
    _, Hq, D = q.shape
    Hkv = k.shape[1]
    dt = dtype_code(x.dtype)
    L = lib()
    ws, nb = _ws(L.dl_qkv_rope_workspace_size(T, H, Hq, Hkv, D, dt), ws, x.device)
    _check(L.dl_qkv_rope(_p(x), _p(w_q), _p(w_k), _p(w_v), _p(positions), _p(cos_sin),
                         cos_sin.shape[0], _p(q), _p(k), _p(v), T, H, Hq, Hkv, D, dt, _p(ws), nb,
                         _stream()))


def dl_qkv_rope_cache(x, w_q, w_k, w_v, positions, cos_sin, q, k, v, seq_of_token, block_table,
                      k_cache, v_cache, Hkv=None, ws=None, k_scale=None, v_scale=None):
    """k, v: [T, Hkv, D] tensors, or both None (K/V then go to the cache only;
    pass Hkv)."""
    T, H = x.shape
    _, Hq, D = q.shape
    Hkv = k.shape[1] if k is not None else Hkv
    dt = dtype_code(x.dtype)
    L = lib()
    ws, nb = _ws(L.dl_qkv_rope_workspace_size(T, H, Hq, Hkv, D, dt), ws, x.device)
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(L.dl_qkv_rope_cache(_p(x), _p(w_q), _p(w_k), _p(w_v), _p(positions), _p(cos_sin),
                               cos_sin.shape[0], _p(q), _p(k), _p(v), _p(seq_of_token),
                               _p(block_table), block_table.shape[1], ctypes.byref(c), T, H, Hq,
                               Hkv, D, k_cache.shape[2], dt, _p(ws), nb, _stream()))


def dl_reshape_and_cache(k, v, seq_of_token, positions, block_table, k_cache, v_cache,
                         k_scale=None, v_scale=None):
    T, Hkv, D = k.shape
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(lib().dl_reshape_and_cache(_p(k), _p(v), _p(seq_of_token), _p(positions),
                                      _p(block_table), block_table.shape[1], ctypes.byref(c), T,
                                      Hkv, D, k_cache.shape[2], dtype_code(k.dtype), _stream()))


def dl_attn_prefill(q, k, v, cu_seqlens, max_seqlen: int, out, scale=None):
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = cu_seqlens.shape[0] - 1
    scale = 0.0 if scale is None else scale       # <= 0: the library's 1/sqrt(D)
    _check(lib().dl_attn_prefill(_p(q), _p(k), _p(v), _p(cu_seqlens), B, T, max_seqlen, Hq, Hkv,
                                 D, scale, _p(out), dtype_code(q.dtype), _stream()))


def dl_attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len: int,
                         out, scale=None, ws=None, k_scale=None, v_scale=None):
    B, Hq, D = q.shape
    Hkv, BS = k_cache.shape[1], k_cache.shape[2]
    scale = 0.0 if scale is None else scale       # <= 0: the library's 1/sqrt(D)
    L = lib()
    ws, nb = _ws(L.dl_attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, BS), ws,
                 q.device)
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(L.dl_attn_decode_paged(_p(q), ctypes.byref(c), _p(block_table), block_table.shape[1],
                                  _p(context_lens), max_context_len, B, Hq, Hkv, D, BS, scale,
                                  _p(out), dtype_code(q.dtype), _p(ws), nb, _stream()))


def dl_attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, context_lens,
                                 max_context_len: int, out, scale=None, k_scale=None,
                                 v_scale=None):
    """dl_attn_decode_paged with the library's fixed device scratch: no
    workspace is passed and nothing is allocated."""
    B, Hq, D = q.shape
    Hkv, BS = k_cache.shape[1], k_cache.shape[2]
    scale = 0.0 if scale is None else scale       # <= 0: the library's 1/sqrt(D)
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(lib().dl_attn_decode_paged_noalloc(_p(q), ctypes.byref(c), _p(block_table),
                                              block_table.shape[1], _p(context_lens),
                                              max_context_len, B, Hq, Hkv, D, BS, scale, _p(out),
                                              dtype_code(q.dtype), _stream()))


def dl_attn_paged_qlens(q, k_cache, v_cache, block_table, cu_q_lens, context_lens,
                        max_q_len: int, max_context_len: int, out, scale=None, ws=None):
    """q, out [Tq, Hq, D] packed by cu_q_lens [B+1]; the new tokens are the
    last q_len of each sequence's context_lens cached positions."""
    Tq, Hq, D = q.shape
    Hkv, BS = k_cache.shape[1], k_cache.shape[2]
    B = cu_q_lens.shape[0] - 1
    scale = 0.0 if scale is None else scale       # <= 0: the library's 1/sqrt(D)
    L = lib()
    ws, nb = _ws(L.dl_attn_paged_qlens_workspace_size(B, Tq, Hq, Hkv, D, max_q_len,
                                                      max_context_len, BS), ws, q.device)
    c = _cache(k_cache, v_cache)
    _check(L.dl_attn_paged_qlens(_p(q), ctypes.byref(c), _p(block_table), block_table.shape[1],
                                 _p(cu_q_lens), _p(context_lens), B, Tq, max_q_len,
                                 max_context_len, Hq, Hkv, D, BS, scale, _p(out),
                                 dtype_code(q.dtype), _p(ws), nb, _stream()))


def dl_linear(x, w, out, ws=None):
    M, K = x.shape
    N = w.shape[0]
    dt = dtype_code(x.dtype)
    L = lib()
    ws, nb = _ws(L.dl_linear_workspace_size(M, N, K, dt), ws, x.device)
    _check(L.dl_linear(_p(x), _p(w), _p(out), M, N, K, dt, _p(ws), nb, _stream()))


def dl_ffn_swiglu(x, w_gate, w_up, w_down, out, residual=None, ws=None):
    T, H = x.shape
    I = w_gate.shape[0]
    dt = dtype_code(x.dtype)
    L = lib()
    ws, nb = _ws(L.dl_ffn_workspace_size(T, H, I, dt), ws, x.device)
    _check(L.dl_ffn_swiglu(_p(x), _p(w_gate), _p(w_up), _p(w_down), _p(residual), _p(out), T, H,
                           I, dt, _p(ws), nb, _stream()))


def dl_gate_up_silu(x, w_gate, w_up, a, ws=None):
    T, H = x.shape
    I = w_gate.shape[0]
    dt = dtype_code(x.dtype)
    L = lib()
    ws, nb = _ws(L.dl_gate_up_silu_workspace_size(T, H, I, dt), ws, x.device)
    _check(L.dl_gate_up_silu(_p(x), _p(w_gate), _p(w_up), _p(a), T, H, I, dt, _p(ws), nb,
                             _stream()))


def dl_down_residual(a, w_down, out, residual=None, ws=None):
    T, I = a.shape
    H = w_down.shape[0]
    dt = dtype_code(a.dtype)
    L = lib()
    ws, nb = _ws(L.dl_down_residual_workspace_size(T, H, I, dt), ws, a.device)
    _check(L.dl_down_residual(_p(a), _p(w_down), _p(residual), _p(out), T, H, I, dt, _p(ws), nb,
                              _stream()))


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

WEIGHT_NAMES = ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd")


def make_dims(hidden, n_q_heads, n_kv_heads, head_dim, intermediate, block_size, rms_eps,
              dtype: torch.dtype) -> LayerDims:
    return LayerDims(hidden, n_q_heads, n_kv_heads, head_dim, intermediate, block_size, rms_eps,
                     dtype_code(dtype))


def make_weights(w: dict) -> LayerWeights:
    return LayerWeights(*[_p(w[n]) for n in WEIGHT_NAMES])


def dl_layer_workspace_size(dims: LayerDims, max_tokens, max_batch, max_seqlen, max_context_len,
                            mode=DL_FUSED) -> int:
    return lib().dl_layer_workspace_size(ctypes.byref(dims), max_tokens, max_batch, max_seqlen,
                                         max_context_len, mode)


def dl_layer_prefill(dims: LayerDims, weights: dict, cos_sin, hidden_in, hidden_out, positions,
                     seq_of_token, cu_seqlens, max_seqlen, k_cache, v_cache, block_table,
                     mode=DL_FUSED, ws=None, k_scale=None, v_scale=None):
    T = hidden_in.shape[0]
    B = cu_seqlens.shape[0] - 1
    L = lib()
    if ws is None:
        n = L.dl_layer_workspace_size(ctypes.byref(dims), T, B, max_seqlen, 0, mode)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=hidden_in.device)
    wts = make_weights(weights)
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(L.dl_layer_prefill(ctypes.byref(dims), ctypes.byref(wts), _p(cos_sin),
                              cos_sin.shape[0], _p(hidden_in), _p(hidden_out), _p(positions),
                              _p(seq_of_token), _p(cu_seqlens), B, T, max_seqlen, ctypes.byref(c),
                              _p(block_table), block_table.shape[1], mode, _p(ws),
                              ws.numel() * ws.element_size(), _stream()))


def dl_layer_decode(dims: LayerDims, weights: dict, cos_sin, hidden_in, hidden_out, positions,
                    context_lens, max_context_len, k_cache, v_cache, block_table, mode=DL_FUSED,
                    ws=None, k_scale=None, v_scale=None):
    B = hidden_in.shape[0]
    L = lib()
    if ws is None:
        n = L.dl_layer_workspace_size(ctypes.byref(dims), B, B, 0, max_context_len, mode)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=hidden_in.device)
    wts = make_weights(weights)
    c = _cache(k_cache, v_cache, k_scale, v_scale)
    _check(L.dl_layer_decode(ctypes.byref(dims), ctypes.byref(wts), _p(cos_sin), cos_sin.shape[0],
                             _p(hidden_in), _p(hidden_out), _p(positions), _p(context_lens),
                             max_context_len, B, ctypes.byref(c), _p(block_table),
                             block_table.shape[1], mode, _p(ws), ws.numel() * ws.element_size(),
                             _stream()))


def dl_layer_decode_qlens(dims: LayerDims, weights: dict, cos_sin, hidden_in, hidden_out,
                          positions, seq_of_token, cu_q_lens, context_lens, max_q_len: int,
                          max_context_len: int, k_cache, v_cache, block_table, ws=None):
    T = hidden_in.shape[0]
    B = cu_q_lens.shape[0] - 1
    L = lib()
    if ws is None:
        n = L.dl_layer_decode_qlens_workspace_size(ctypes.byref(dims), T, B, max_q_len,
                                                   max_context_len)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=hidden_in.device)
    wts = make_weights(weights)
    c = _cache(k_cache, v_cache)
    _check(L.dl_layer_decode_qlens(ctypes.byref(dims), ctypes.byref(wts), _p(cos_sin),
                                   cos_sin.shape[0], _p(hidden_in), _p(hidden_out), _p(positions),
                                   _p(seq_of_token), _p(cu_q_lens), _p(context_lens), B, T,
                                   max_q_len, max_context_len, ctypes.byref(c), _p(block_table),
                                   block_table.shape[1], DL_FUSED, _p(ws),
                                   ws.numel() * ws.element_size(), _stream()))


class DecodeGraph:
    """dl_layer_decode recorded once (dl_layer_decode_graph_create) and
    replayed with dl_graph_launch.  The tensors passed here are baked into
    the graph: update their contents in place between launches.  Capture and
    replay run on `stream` (a torch.cuda.Stream, not the default stream)."""

    def __init__(self, dims: LayerDims, weights: dict, cos_sin, hidden_in, hidden_out, positions,
                 context_lens, max_context_len: int, k_cache, v_cache, block_table, stream,
                 ws=None, k_scale=None, v_scale=None):
        B = hidden_in.shape[0]
        L = lib()
        if ws is None:
            n = L.dl_layer_workspace_size(ctypes.byref(dims), B, B, 0, max_context_len, DL_FUSED)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=hidden_in.device)
        self._keep = (dims, weights, cos_sin, hidden_in, hidden_out, positions, context_lens,
                      k_cache, v_cache, block_table, ws, k_scale, v_scale)
        self.stream = stream
        self._wts = make_weights(weights)
        self._cache = _cache(k_cache, v_cache, k_scale, v_scale)
        h = _vp()
        _check(L.dl_layer_decode_graph_create(
            ctypes.byref(dims), ctypes.byref(self._wts), _p(cos_sin), cos_sin.shape[0],
            _p(hidden_in), _p(hidden_out), _p(positions), _p(context_lens), max_context_len, B,
            ctypes.byref(self._cache), _p(block_table), block_table.shape[1], _p(ws),
            ws.numel() * ws.element_size(), stream.cuda_stream, ctypes.byref(h)))
        self._h = h

    def launch(self):
        _check(lib().dl_graph_launch(self._h, self.stream.cuda_stream))

    def close(self):
        if self._h:
            _check(lib().dl_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
