"""CPU oracle for the Llama-style decoder layer -- TEST INFRASTRUCTURE ONLY.

This package wraps ``orc.c`` (plain C, fp64 accumulation, OpenMP) through
ctypes.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the GPU library never does, and the two share no
code.  Inputs and outputs are numpy float32 arrays (bf16 data is carried as
the fp32 value it represents) and int32 index arrays.

Every function cites the page passage it follows in ``orc.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB = os.path.join(_HERE, "liborc.so")

EXACT = 0
BF16 = 1
BF16_UNFUSED = 2

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile orc.c into liborc.so with gcc (-O3, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            _lib = ctypes.CDLL(_LIB)
            _declare(_lib)
    return _lib


_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i = ctypes.c_int
_d = ctypes.c_double


class Dims(ctypes.Structure):
    _fields_ = [("hidden", _i), ("n_q_heads", _i), ("n_kv_heads", _i),
                ("head_dim", _i), ("intermediate", _i), ("block_size", _i),
                ("rms_eps", _d), ("rope_theta", _d)]


class Weights(ctypes.Structure):
    _fields_ = [(n, _f32p) for n in ("ln1", "wq", "wk", "wv", "wo", "ln2",
                                      "wg", "wu", "wd")]


def _declare(L):
    L.orc_bf16_round.argtypes = [ctypes.c_float]
    L.orc_bf16_round.restype = ctypes.c_float
    L.orc_round_bf16_array.argtypes = [_f32p, ctypes.c_int64]
    L.orc_rmsnorm.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _i, _i, _d, _i]
    L.orc_linear.argtypes = [_f32p, _f32p, _f32p, _i, _i, _i, _i]
    L.orc_rope.argtypes = [_f32p, _i32p, _i, _i, _i, _d, _i]
    L.orc_qkv_rope.argtypes = [_f32p, _f32p, _f32p, _f32p, _i32p, _d, _f32p,
                               _f32p, _f32p, _i, _i, _i, _i, _i, _i]
    L.orc_reshape_and_cache.argtypes = [_f32p, _f32p, _i32p, _i32p, _i32p, _i,
                                        _f32p, _f32p, _i, _i, _i, _i]
    L.orc_attn_prefill.argtypes = [_f32p, _f32p, _f32p, _i32p, _i, _i, _i, _i,
                                   _d, _f32p, _i]
    L.orc_attn_decode_paged.argtypes = [_f32p, _f32p, _f32p, _i32p, _i, _i32p,
                                        _i, _i, _i, _i, _i, _d, _f32p, _i]
    L.orc_attn_paged_qlens.argtypes = [_f32p, _f32p, _f32p, _i32p, _i, _i32p, _i32p, _i,
                                       _i, _i, _i, _i, _d, _f32p, _i]
    L.orc_attn_decode_contig.argtypes = [_f32p, _f32p, _f32p, _i, _i32p, _i, _i,
                                         _i, _i, _d, _f32p, _i]
    L.orc_swiglu.argtypes = [_f32p, _f32p, _f32p, _f32p, _i, _i, _i, _i]
    L.orc_swiglu_parts.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i, _i,
                                   _i, _i]
    L.orc_attn_row.argtypes = [_f32p, _f32p, _f32p, _i, _i, _d, _i, _f32p, _f32p, _f32p]
    L.orc_down_residual.argtypes = [_f32p, _f32p, _f32p, _f32p, _i, _i, _i]
    L.orc_ffn.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i, _i, _i, _i]
    L.orc_layer_prefill.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                    _f32p, _f32p, _f32p, _i32p, _i32p, _i32p, _i,
                                    _i, _f32p, _f32p, _i32p, _i, _i]
    L.orc_layer_decode.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                   _f32p, _f32p, _f32p, _i32p, _i, _f32p, _f32p,
                                   _i32p, _i, _i]
    L.orc_kv_quant_rows.argtypes = [_f32p, ctypes.c_int64, _i, _i8p, _f32p]
    L.orc_reshape_and_cache_q8.argtypes = [_f32p, _f32p, _i32p, _i32p, _i32p, _i,
                                           _i8p, _i8p, _f32p, _f32p, _i, _i, _i, _i]
    L.orc_attn_decode_paged_q8.argtypes = [_f32p, _i8p, _i8p, _f32p, _f32p, _i32p,
                                           _i, _i32p, _i, _i, _i, _i, _i, _d, _f32p,
                                           _i]
    L.orc_layer_prefill_q8.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                       _f32p, _f32p, _f32p, _i32p, _i32p, _i32p, _i,
                                       _i, _i8p, _i8p, _f32p, _f32p, _i32p, _i, _i]
    L.orc_layer_decode_q8.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                      _f32p, _f32p, _f32p, _i32p, _i, _i8p, _i8p,
                                      _f32p, _f32p, _i32p, _i, _i]
    L.orc_layer_decode_qlens.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                         _f32p, _f32p, _f32p, _i32p, _i32p, _i32p, _i32p, _i,
                                         _i, _f32p, _f32p, _i32p, _i, _i]
    L.orc_kv_cache_bytes.argtypes = [_i, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, _i]
    L.orc_kv_cache_bytes.restype = _d


def _f(a, shape=None):
    """Contiguous float32 view (copy only if needed) and its pointer."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None:
        assert a.size == int(np.prod(shape)), (a.shape, shape)
    return a


def _p(a):
    if a is None:
        return None
    if a.dtype == np.float32:
        return a.ctypes.data_as(_f32p)
    if a.dtype == np.int32:
        return a.ctypes.data_as(_i32p)
    if a.dtype == np.int8:
        return a.ctypes.data_as(_i8p)
    raise TypeError(a.dtype)


def _ii(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# ---------------------------------------------------------------------------
# step functions
# ---------------------------------------------------------------------------

def bf16_round(x):
    """fp32 -> nearest bf16 (ties to even), returned as float32."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    lib().orc_round_bf16_array(_p(out), out.size)
    return out


def rmsnorm(x, gamma, eps=1e-5, resid=None, mode=EXACT):
    """Returns n (and h when resid is given).  x, resid [T, H]."""
    x = _f(x)
    T, H = x.shape
    g = _f(gamma)
    out = np.empty_like(x)
    if resid is None:
        lib().orc_rmsnorm(_p(x), None, None, _p(g), _p(out), T, H, eps, mode)
        return out
    r = _f(resid)
    h = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(r), _p(h), _p(g), _p(out), T, H, eps, mode)
    return out, h


def linear(x, w, round_bf16=False):
    x, w = _f(x), _f(w)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((M, N), np.float32)
    lib().orc_linear(_p(x), _p(w), _p(y), M, N, K, int(round_bf16))
    return y


def rope(u, pos, theta, round_bf16=False):
    """u [T, nh, D] -> rotated copy."""
    u = np.array(u, dtype=np.float32, copy=True, order="C")
    T, nh, D = u.shape
    lib().orc_rope(_p(u), _p(_ii(pos)), T, nh, D, theta, int(round_bf16))
    return u


def qkv_rope(x, wq, wk, wv, pos, theta, Hq, Hkv, D, mode=EXACT):
    x = _f(x)
    T, H = x.shape
    q = np.empty((T, Hq, D), np.float32)
    k = np.empty((T, Hkv, D), np.float32)
    v = np.empty((T, Hkv, D), np.float32)
    lib().orc_qkv_rope(_p(x), _p(_f(wq)), _p(_f(wk)), _p(_f(wv)), _p(_ii(pos)),
                       theta, _p(q), _p(k), _p(v), T, H, Hq, Hkv, D, mode)
    return q, k, v


def reshape_and_cache(k, v, seq_of_token, pos, block_table, k_cache, v_cache):
    """Writes into k_cache / v_cache [nb, Hkv, BS, D] in place (float32)."""
    k, v = _f(k), _f(v)
    T, Hkv, D = k.shape
    bt = _ii(block_table)
    assert k_cache.dtype == np.float32 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.float32 and v_cache.flags.c_contiguous
    BS = k_cache.shape[2]
    lib().orc_reshape_and_cache(_p(k), _p(v), _p(_ii(seq_of_token)), _p(_ii(pos)),
                                _p(bt), bt.shape[1], _p(k_cache), _p(v_cache),
                                T, Hkv, D, BS)


def _cache_out(a, dtype, name):
    assert a.dtype == dtype and a.flags.c_contiguous, name


def kv_quant_rows(x):
    """INT8 per-row quantisation of x [..., D] -> (codes int8 [..., D], scales [...])."""
    x = _f(x)
    D = x.shape[-1]
    R = x.size // D
    codes = np.empty(x.shape, np.int8)
    scales = np.empty(x.shape[:-1], np.float32)
    lib().orc_kv_quant_rows(_p(x), R, D, _p(codes), _p(scales))
    return codes, scales


def reshape_and_cache_q8(k, v, seq_of_token, pos, block_table, k_codes, v_codes,
                         k_scale, v_scale):
    """Quantising cache write, in place: codes int8 [nb, Hkv, BS, D], scales
    float32 [nb, Hkv, BS]."""
    k, v = _f(k), _f(v)
    T, Hkv, D = k.shape
    bt = _ii(block_table)
    for a, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _cache_out(a, np.int8, n)
    for a, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _cache_out(a, np.float32, n)
    BS = k_codes.shape[2]
    lib().orc_reshape_and_cache_q8(_p(k), _p(v), _p(_ii(seq_of_token)), _p(_ii(pos)),
                                   _p(bt), bt.shape[1], _p(k_codes), _p(v_codes),
                                   _p(k_scale), _p(v_scale), T, Hkv, D, BS)


def attn_prefill(q, k, v, cu_seqlens, scale=None, mode=EXACT):
    q, k, v = _f(q), _f(k), _f(v)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    cu = _ii(cu_seqlens)
    B = cu.size - 1
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.empty_like(q)
    lib().orc_attn_prefill(_p(q), _p(k), _p(v), _p(cu), B, Hq, Hkv, D, scale,
                           _p(out), mode)
    return out


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, scale=None,
                      mode=EXACT):
    q = _f(q)
    B, Hq, D = q.shape
    kc, vc = _f(k_cache), _f(v_cache)
    Hkv, BS = kc.shape[1], kc.shape[2]
    bt = _ii(block_table)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.empty_like(q)
    lib().orc_attn_decode_paged(_p(q), _p(kc), _p(vc), _p(bt), bt.shape[1],
                                _p(_ii(context_lens)), B, Hq, Hkv, D, BS, scale,
                                _p(out), mode)
    return out


def attn_decode_paged_q8(q, k_codes, v_codes, k_scale, v_scale, block_table,
                         context_lens, scale=None, mode=EXACT):
    q = _f(q)
    B, Hq, D = q.shape
    kq = np.ascontiguousarray(k_codes, dtype=np.int8)
    vq = np.ascontiguousarray(v_codes, dtype=np.int8)
    ks, vs = _f(k_scale), _f(v_scale)
    Hkv, BS = kq.shape[1], kq.shape[2]
    bt = _ii(block_table)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.empty_like(q)
    lib().orc_attn_decode_paged_q8(_p(q), _p(kq), _p(vq), _p(ks), _p(vs), _p(bt),
                                   bt.shape[1], _p(_ii(context_lens)), B, Hq, Hkv, D,
                                   BS, scale, _p(out), mode)
    return out


def attn_paged_qlens(q, k_cache, v_cache, block_table, cu_q, context_lens, scale=None,
                     mode=EXACT):
    """q [Tq, Hq, D] packed by cu_q [B+1]; the new tokens are the last
    cu_q[b+1]-cu_q[b] of the context_lens[b] cached positions."""
    q = _f(q)
    Tq, Hq, D = q.shape
    kc, vc = _f(k_cache), _f(v_cache)
    Hkv, BS = kc.shape[1], kc.shape[2]
    bt = _ii(block_table)
    cu = _ii(cu_q)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.empty_like(q)
    lib().orc_attn_paged_qlens(_p(q), _p(kc), _p(vc), _p(bt), bt.shape[1], _p(cu),
                               _p(_ii(context_lens)), cu.size - 1, Hq, Hkv, D, BS, scale,
                               _p(out), mode)
    return out


def attn_decode_contig(q, k_cache, v_cache, context_lens, scale=None, mode=EXACT):
    """k_cache / v_cache [B, Hkv, S, D]."""
    q = _f(q)
    B, Hq, D = q.shape
    kc, vc = _f(k_cache), _f(v_cache)
    Hkv, S = kc.shape[1], kc.shape[2]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = np.empty_like(q)
    lib().orc_attn_decode_contig(_p(q), _p(kc), _p(vc), S, _p(_ii(context_lens)),
                                 B, Hq, Hkv, D, scale, _p(out), mode)
    return out


def swiglu(x, wg, wu, mode=EXACT):
    x = _f(x)
    M, H = x.shape
    I = wg.shape[0]
    a = np.empty((M, I), np.float32)
    lib().orc_swiglu(_p(x), _p(_f(wg)), _p(_f(wu)), _p(a), M, H, I, mode)
    return a


def swiglu_parts(x, wg, wu, mode=EXACT):
    """(g, u, silu(g), a), each [M, I], as stored in the given mode."""
    x = _f(x)
    M, H = x.shape
    I = wg.shape[0]
    g, u, sg, a = (np.empty((M, I), np.float32) for _ in range(4))
    lib().orc_swiglu_parts(_p(x), _p(_f(wg)), _p(_f(wu)), _p(g), _p(u), _p(sg), _p(a), M, H,
                           I, mode)
    return g, u, sg, a


def attn_row(q, k, v, scale=None, mode=EXACT):
    """One query row q [D] over keys k [n, D] and values v [n, D]:
    (scores [n], probabilities [n], output [D]) as stored in the given mode."""
    q, k, v = _f(q), _f(k), _f(v)
    D = q.shape[-1]
    n = k.shape[0]
    assert k.shape == (n, D) and v.shape == (n, D) and q.size == D
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    s = np.empty(n, np.float32)
    p = np.empty(n, np.float32)
    o = np.empty(D, np.float32)
    lib().orc_attn_row(_p(q), _p(k), _p(v), n, D, scale, mode, _p(s), _p(p), _p(o))
    return s, p, o


def down_residual(a, wd, resid=None):
    a = _f(a)
    M, I = a.shape
    H = wd.shape[0]
    y = np.empty((M, H), np.float32)
    lib().orc_down_residual(_p(a), _p(_f(wd)), _p(None if resid is None else _f(resid)),
                            _p(y), M, H, I)
    return y


def ffn(x, wg, wu, wd, resid=None, mode=EXACT):
    x = _f(x)
    M, H = x.shape
    I = wg.shape[0]
    y = np.empty((M, H), np.float32)
    r = None if resid is None else _f(resid)
    lib().orc_ffn(_p(x), _p(_f(wg)), _p(_f(wu)), _p(_f(wd)), _p(r), _p(y), M, H, I,
                  mode)
    return y


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

_WNAMES = ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd")


def _pack(dims, weights):
    d = Dims(dims["hidden"], dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"],
             dims["intermediate"], dims["block_size"], dims["rms_eps"],
             dims["rope_theta"])
    arrs = {n: _f(weights[n]) for n in _WNAMES}
    w = Weights(*[_p(arrs[n]) for n in _WNAMES])
    return d, w, arrs


def layer_prefill(dims, weights, x, pos, seq_of_token, cu_seqlens, k_cache=None,
                  v_cache=None, block_table=None, mode=EXACT):
    """Returns (y, h).  Caches (float32, [nb, Hkv, BS, D]) updated in place."""
    d, w, keep = _pack(dims, weights)
    x = _f(x)
    T, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    cu = _ii(cu_seqlens)
    bt = _ii(block_table) if block_table is not None else None
    lib().orc_layer_prefill(ctypes.byref(d), ctypes.byref(w), _p(x), _p(y), _p(h),
                            _p(_ii(pos)), _p(_ii(seq_of_token)), _p(cu), cu.size - 1,
                            T, _p(k_cache), _p(v_cache), _p(bt),
                            0 if bt is None else bt.shape[1], mode)
    del keep
    return y, h


def layer_decode(dims, weights, x, context_lens, k_cache, v_cache, block_table,
                 mode=EXACT):
    d, w, keep = _pack(dims, weights)
    x = _f(x)
    B, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    bt = _ii(block_table)
    assert k_cache.dtype == np.float32 and k_cache.flags.c_contiguous
    lib().orc_layer_decode(ctypes.byref(d), ctypes.byref(w), _p(x), _p(y), _p(h),
                           _p(_ii(context_lens)), B, _p(k_cache), _p(v_cache), _p(bt),
                           bt.shape[1], mode)
    del keep
    return y, h


def layer_decode_qlens(dims, weights, x, pos, seq_of_token, cu_q, context_lens, k_cache,
                       v_cache, block_table, mode=EXACT):
    """New tokens (packed by cu_q) appended to cached sequences; caches
    (float32) updated in place.  Returns (y, h)."""
    d, w, keep = _pack(dims, weights)
    x = _f(x)
    T, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    cu = _ii(cu_q)
    bt = _ii(block_table)
    assert k_cache.dtype == np.float32 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.float32 and v_cache.flags.c_contiguous
    lib().orc_layer_decode_qlens(ctypes.byref(d), ctypes.byref(w), _p(x), _p(y), _p(h),
                                 _p(_ii(pos)), _p(_ii(seq_of_token)), _p(cu),
                                 _p(_ii(context_lens)), cu.size - 1, T, _p(k_cache),
                                 _p(v_cache), _p(bt), bt.shape[1], mode)
    del keep
    return y, h


def layer_prefill_q8(dims, weights, x, pos, seq_of_token, cu_seqlens, k_codes,
                     v_codes, k_scale, v_scale, block_table, mode=EXACT):
    """layer_prefill with an INT8 cache (updated in place).  Returns (y, h)."""
    d, w, keep = _pack(dims, weights)
    x = _f(x)
    T, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    cu = _ii(cu_seqlens)
    bt = _ii(block_table)
    for a, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _cache_out(a, np.int8, n)
    for a, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _cache_out(a, np.float32, n)
    lib().orc_layer_prefill_q8(ctypes.byref(d), ctypes.byref(w), _p(x), _p(y), _p(h),
                               _p(_ii(pos)), _p(_ii(seq_of_token)), _p(cu), cu.size - 1,
                               T, _p(k_codes), _p(v_codes), _p(k_scale), _p(v_scale),
                               _p(bt), bt.shape[1], mode)
    del keep
    return y, h


def layer_decode_q8(dims, weights, x, context_lens, k_codes, v_codes, k_scale,
                    v_scale, block_table, mode=EXACT):
    """layer_decode with an INT8 cache (updated in place).  Returns (y, h)."""
    d, w, keep = _pack(dims, weights)
    x = _f(x)
    B, H = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    bt = _ii(block_table)
    for a, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _cache_out(a, np.int8, n)
    for a, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _cache_out(a, np.float32, n)
    lib().orc_layer_decode_q8(ctypes.byref(d), ctypes.byref(w), _p(x), _p(y), _p(h),
                              _p(_ii(context_lens)), B, _p(k_codes), _p(v_codes),
                              _p(k_scale), _p(v_scale), _p(bt), bt.shape[1], mode)
    del keep
    return y, h


def kv_cache_bytes(layers, seq, batch, d_kv, elem_bytes):
    return lib().orc_kv_cache_bytes(layers, seq, batch, d_kv, elem_bytes)
