"""Seeded synthetic workloads for the decoder layer (tests and benchmark).

This module only draws numbers and lays out indices; it computes nothing of
the layer itself.  Both the GPU path and the CPU oracle are fed from here.

Recipe (shapes from the five workload configurations):
  * every random tensor comes from numpy default_rng(SeedSequence(
    [config_id, tensor_id, step, block])), one stream per 2^22-element block
    of the flattened tensor, so any tensor can be regenerated alone;
  * the seven projection matrices are N(0, 0.02^2); RMSNorm gammas are 1
    (unit tests may ask for U(0.5, 1.5) so a dropped gamma is visible);
  * hidden states are N(0, 1); in bf16 configurations every draw is rounded
    to the nearest bf16 value (ties to even) and carried as float32;
  * packed prefill: positions restart at 0 in every sequence;
  * paged cache: the pool holds the blocks every sequence needs plus at least
    8 spare blocks; physical ids are a seeded permutation of the pool taken in
    (sequence, logical block) order; unused table entries are -1; every slot
    that is not written holds a NaN sentinel;
  * decode with no prefill of its own (7B and 70B decode): earlier positions
    hold synthetic K/V ~ N(0, H * 0.02^2), the variance W_k x would have;
  * INT8 caches: codes uniform over the integers -127 .. 127 and row scales
    uniform in [2.5, 3.5] * sigma / 127 (sigma the K/V spread above), drawn
    directly; unwritten rows hold code -128 (never a quantiser output) and a
    NaN scale.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass, field

import numpy as np

# tensor ids of the seed sequence
T_LN1, T_WQ, T_WK, T_WV, T_WO, T_LN2, T_WG, T_WU, T_WD = range(9)
T_X, T_LENS, T_PERM, T_KCACHE, T_VCACHE, T_CTX, T_MISC = 20, 21, 22, 23, 24, 25, 26
T_KCODES, T_VCODES, T_KSCALE, T_VSCALE = 27, 28, 29, 30

BF16_SENTINEL = np.uint16(0x7FC1)          # quiet NaN with a payload
F32_SENTINEL = np.uint32(0x7FC00001)
CODE_SENTINEL = np.int8(-128)


@dataclass(frozen=True)
class LayerConfig:
    config_id: int
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    block_size: int
    rope_theta: float
    dtype: str                      # "bf16" or "f32"
    rms_eps: float = 1e-5
    prefill_lens: tuple = ()        # fixed prefill lengths, or ()
    prefill_uniform: tuple = ()     # (batch, lo, hi): ragged lengths U{lo..hi}
    decode_steps: int = 0           # decode steps after the config's own prefill
    decode_batch: int = 0           # decode without prefill: batch
    decode_ctx: tuple = ()          # (lo, hi) uniform context lengths
    extra: dict = field(default_factory=dict)

    def dims(self) -> dict:
        return dict(hidden=self.hidden, n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, intermediate=self.intermediate,
                    block_size=self.block_size, rms_eps=self.rms_eps,
                    rope_theta=self.rope_theta)


CONFIGS = {
    1: LayerConfig(1, "tiny-fp32", 256, 4, 4, 64, 688, 16, 1e4, "f32",
                   prefill_lens=(32,), decode_steps=8),
    2: LayerConfig(2, "llama2-7b-prefill", 4096, 32, 32, 128, 11008, 128, 1e4, "bf16",
                   prefill_lens=(2048,)),
    3: LayerConfig(3, "llama2-7b-decode", 4096, 32, 32, 128, 11008, 128, 1e4, "bf16",
                   decode_batch=64, decode_ctx=(128, 4096)),
    4: LayerConfig(4, "llama3-8b-gqa", 4096, 32, 8, 128, 14336, 128, 5e5, "bf16",
                   prefill_uniform=(8, 256, 1024), decode_steps=128),
    5: LayerConfig(5, "llama-70b-decode", 8192, 64, 8, 128, 28672, 128, 1e4, "bf16",
                   extra={"cases": ((4, 4096), (1, 32768))}),
}


def rng(config_id: int, tensor_id: int, step: int = 0, chunk: int = -1) -> np.random.Generator:
    key = [config_id, tensor_id, step] if chunk < 0 else [config_id, tensor_id, step, chunk]
    return np.random.default_rng(np.random.SeedSequence(key))


_CHUNK = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def _standard_normal(config_id: int, tensor_id: int, step: int, shape) -> np.ndarray:
    """N(0,1) float32 draws; element block c (of 2^22) comes from its own
    stream rng(config_id, tensor_id, step, c), so blocks fill in parallel."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1)

    def fill(c):
        s = c * _CHUNK
        e = min(flat.size, s + _CHUNK)
        flat[s:e] = rng(config_id, tensor_id, step, c).standard_normal(e - s, dtype=np.float32)

    list(_pool().map(fill, range((flat.size + _CHUNK - 1) // _CHUNK)))
    return out


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each float32, returned as float32.
    Works in place on a private float32 copy, in chunks to bound temporaries."""
    out = np.array(a, dtype=np.float32, copy=True, order="C")
    u = out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s:s + step]
        nan = np.isnan(c.view(np.float32))
        lsb = (c >> np.uint32(16)) & np.uint32(1)
        c += np.uint32(0x7FFF)
        c += lsb
        c &= np.uint32(0xFFFF0000)
        if nan.any():
            c[nan] = np.uint32(0x7FC00000)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16 values."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _round_bf16_inplace(a: np.ndarray) -> np.ndarray:
    """In-place nearest-bf16 rounding (ties to even) of finite float32 draws,
    in parallel blocks."""
    u = a.reshape(-1).view(np.uint32)

    def rnd(c):
        v = u[c * _CHUNK:(c + 1) * _CHUNK]
        lsb = (v >> np.uint32(16)) & np.uint32(1)
        v += np.uint32(0x7FFF)
        v += lsb
        v &= np.uint32(0xFFFF0000)

    list(_pool().map(rnd, range((u.size + _CHUNK - 1) // _CHUNK)))
    return a


def _normal(cfg: LayerConfig, tensor_id: int, shape, sigma: float, step: int = 0):
    a = _standard_normal(cfg.config_id, tensor_id, step, shape)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return _round_bf16_inplace(a) if cfg.dtype == "bf16" else a


def weights(cfg: LayerConfig, gamma: str = "ones") -> dict:
    """The layer's nine parameter tensors as float32 arrays."""
    H, Hq, Hkv, D, I = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    w = {
        "wq": _normal(cfg, T_WQ, (Hq * D, H), 0.02),
        "wk": _normal(cfg, T_WK, (Hkv * D, H), 0.02),
        "wv": _normal(cfg, T_WV, (Hkv * D, H), 0.02),
        "wo": _normal(cfg, T_WO, (H, Hq * D), 0.02),
        "wg": _normal(cfg, T_WG, (I, H), 0.02),
        "wu": _normal(cfg, T_WU, (I, H), 0.02),
        "wd": _normal(cfg, T_WD, (H, I), 0.02),
    }
    for name, tid in (("ln1", T_LN1), ("ln2", T_LN2)):
        if gamma == "ones":
            w[name] = np.ones(H, np.float32)
        else:
            g = rng(cfg.config_id, tid).uniform(0.5, 1.5, H).astype(np.float32)
            w[name] = to_bf16_values(g) if cfg.dtype == "bf16" else g
    return w


def hidden(cfg: LayerConfig, T: int, step: int = 0) -> np.ndarray:
    """Residual-stream input [T, H] (float32; bf16 values in bf16 configs)."""
    return _normal(cfg, T_X, (T, cfg.hidden), 1.0, step)


@dataclass
class PrefillBatch:
    lens: np.ndarray          # [B]
    cu_seqlens: np.ndarray    # [B+1]
    positions: np.ndarray     # [T]
    seq_of_token: np.ndarray  # [T]

    @property
    def T(self):
        return int(self.cu_seqlens[-1])

    @property
    def B(self):
        return int(self.lens.size)

    @property
    def max_seqlen(self):
        return int(self.lens.max()) if self.lens.size else 0


def packed(lens) -> PrefillBatch:
    lens = np.asarray(lens, dtype=np.int32)
    cu = np.zeros(lens.size + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens]) if lens.size else \
        np.zeros(0, np.int32)
    seq = np.repeat(np.arange(lens.size, dtype=np.int32), lens)
    return PrefillBatch(lens, cu, pos, seq)


def prefill_batch(cfg: LayerConfig) -> PrefillBatch:
    if cfg.prefill_lens:
        return packed(cfg.prefill_lens)
    B, lo, hi = cfg.prefill_uniform
    return packed(rng(cfg.config_id, T_LENS).integers(lo, hi + 1, B))


def decode_context_lens(cfg: LayerConfig, case: int = 0) -> np.ndarray:
    """Context lengths (counting the new token) for decode without prefill."""
    if cfg.decode_ctx:
        lo, hi = cfg.decode_ctx
        return rng(cfg.config_id, T_CTX).integers(lo, hi + 1, cfg.decode_batch).astype(np.int32)
    B, ctx = cfg.extra["cases"][case]
    return np.full(B, ctx, np.int32)


@dataclass
class BlockTable:
    table: np.ndarray     # [B, max_blocks] int32, -1 where unused
    num_blocks: int


def block_table(cfg: LayerConfig, capacity, spare: int = 8, step: int = 0,
                identity: bool = False) -> BlockTable:
    """Blocks for sequences that will hold up to capacity[b] tokens."""
    BS = cfg.block_size
    capacity = np.asarray(capacity, dtype=np.int64)
    need = (capacity + BS - 1) // BS
    used = int(need.sum())
    pool = used + spare
    ids = np.arange(pool, dtype=np.int32) if identity else \
        rng(cfg.config_id, T_PERM, step).permutation(pool).astype(np.int32)
    maxb = int(need.max()) if need.size else 1
    tab = np.full((capacity.size, max(maxb, 1)), -1, np.int32)
    k = 0
    for b, n in enumerate(need):
        tab[b, :n] = ids[k:k + n]
        k += n
    return BlockTable(tab, pool)


def empty_cache(cfg: LayerConfig, num_blocks: int):
    """Sentinel-filled K and V caches [num_blocks, Hkv, BS, D] as raw bits
    (uint16 for bf16 configs, uint32 for fp32)."""
    shape = (num_blocks, cfg.n_kv_heads, cfg.block_size, cfg.head_dim)
    if cfg.dtype == "bf16":
        return np.full(shape, BF16_SENTINEL, np.uint16), np.full(shape, BF16_SENTINEL, np.uint16)
    return np.full(shape, F32_SENTINEL, np.uint32), np.full(shape, F32_SENTINEL, np.uint32)


def synthetic_cache(cfg: LayerConfig, bt: BlockTable, context_lens, case: int = 0):
    """Caches whose positions 0 .. ctx-2 of every sequence hold synthetic K/V
    (the new token's slot ctx-1 and all other slots keep the sentinel)."""
    kc, vc = empty_cache(cfg, bt.num_blocks)
    BS, Hkv, D = cfg.block_size, cfg.n_kv_heads, cfg.head_dim
    sigma = float(np.sqrt(cfg.hidden) * 0.02)
    for b, n in enumerate(np.asarray(context_lens)):
        prior = int(n) - 1
        if prior <= 0:
            continue
        nblk = (prior + BS - 1) // BS
        for which, cache, tid in ((0, kc, T_KCACHE), (1, vc, T_VCACHE)):
            vals = _standard_normal(cfg.config_id, tid, 1000 * case + b, (nblk * BS, Hkv, D))
            vals *= np.float32(sigma)
            if cfg.dtype == "bf16":
                bits = bf16_bits(_round_bf16_inplace(vals))
            else:
                bits = vals.view(np.uint32)
            bits = bits.reshape(nblk, BS, Hkv, D).transpose(0, 2, 1, 3)
            for j in range(nblk):
                ntok = min(BS, prior - j * BS)
                phys = bt.table[b, j]
                cache[phys, :, :ntok, :] = bits[j, :, :ntok, :]
    return kc, vc


def empty_cache_q8(cfg: LayerConfig, num_blocks: int):
    """Sentinel-filled INT8 cache: codes (k, v) [num_blocks, Hkv, BS, D] int8
    and row scales (k, v) [num_blocks, Hkv, BS] float32."""
    shape = (num_blocks, cfg.n_kv_heads, cfg.block_size, cfg.head_dim)
    return (np.full(shape, CODE_SENTINEL, np.int8), np.full(shape, CODE_SENTINEL, np.int8),
            np.full(shape[:3], np.nan, np.float32), np.full(shape[:3], np.nan, np.float32))


def synthetic_cache_q8(cfg: LayerConfig, bt: BlockTable, context_lens, case: int = 0):
    """INT8 counterpart of synthetic_cache: positions 0 .. ctx-2 of every
    sequence hold drawn codes and scales, everything else the sentinels."""
    kq, vq, ks, vs = empty_cache_q8(cfg, bt.num_blocks)
    BS, Hkv, D = cfg.block_size, cfg.n_kv_heads, cfg.head_dim
    sigma = float(np.sqrt(cfg.hidden) * 0.02)
    for b, n in enumerate(np.asarray(context_lens)):
        prior = int(n) - 1
        if prior <= 0:
            continue
        nblk = (prior + BS - 1) // BS
        for codes, scales, tc, tsc in ((kq, ks, T_KCODES, T_KSCALE), (vq, vs, T_VCODES, T_VSCALE)):
            c = rng(cfg.config_id, tc, 1000 * case + b).integers(
                -127, 128, (nblk, Hkv, BS, D), dtype=np.int16).astype(np.int8)
            sc = (rng(cfg.config_id, tsc, 1000 * case + b).uniform(2.5, 3.5, (nblk, Hkv, BS))
                  * (sigma / 127.0)).astype(np.float32)
            for j in range(nblk):
                ntok = min(BS, prior - j * BS)
                phys = bt.table[b, j]
                codes[phys, :, :ntok] = c[j, :, :ntok]
                scales[phys, :, :ntok] = sc[j, :, :ntok]
    return kq, vq, ks, vs


def cache_to_f32(bits: np.ndarray) -> np.ndarray:
    """Raw cache bits -> float32 values (the oracle's view)."""
    if bits.dtype == np.uint16:
        return bits_to_f32(bits)
    return bits.view(np.float32)
