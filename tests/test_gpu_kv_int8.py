"""INT8 KV cache on the GPU (per-token row scales, quantised on write,
dequantised by the paged decode attention):

  * the quantising cache write gives the oracle's codes and scales bit for
    bit on the same k/v (sentinel rows untouched, invalid table entries
    dropped);
  * paged decode attention over INT8 blocks against the oracle's INT8
    attention, and its independence from the physical block numbering;
  * the whole layer with an INT8 cache: fused equals step by step bit for
    bit, and prefill + decode steps against the oracle's INT8 layer.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from transformer_decoder_layer_residual_amd import binding as dl
from transformer_decoder_layer_residual_amd import inputs as gen
from transformer_decoder_layer_residual_amd.harness import DeviceLayer, cache_dev, i32, to_dev

from _util import (DEV, assert_bf16_close, assert_f32_close, dev_as, dev_i32, host, host_bits)

pytestmark = pytest.mark.gpu

R = np.random.default_rng(2024)
DTYPES = [torch.bfloat16, torch.float32]


def rows_for(T, Hkv, D, dtype):
    """k or v rows with mixed magnitudes, an all-zero row and a one-hot row."""
    x = R.standard_normal((T, Hkv, D)) * R.choice([1e-3, 0.3, 1.0, 40.0], (T, Hkv, 1))
    x[0, 0] = 0.0
    if T > 1:
        x[1, -1] = 0.0
        x[1, -1, 5] = -2.5
    x = x.astype(np.float32)
    return oracle.bf16_round(x) if dtype == torch.bfloat16 else x


def q8_dev(host_cache):
    return tuple(cache_dev(a) for a in host_cache)


def q8_host(dev_cache):
    kq, vq, ks, vs = dev_cache
    return (kq.cpu().numpy(), vq.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy())


def assert_q8_equal(got, want, what):
    for g, w, name in zip(got, want, ("k codes", "v codes", "k scales", "v scales")):
        if g.dtype == np.float32:
            same = g.view(np.uint32) == w.view(np.uint32)
        else:
            same = g == w
        assert same.all(), f"{what}: {int((~same).sum())} {name} differ from the oracle"


@pytest.mark.parametrize("cfg_id,decode", [(1, False), (1, True), (4, False), (4, True)])
def test_reshape_and_cache_q8_bit_exact(cfg_id, decode):
    cfg = gen.CONFIGS[cfg_id]
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Hkv, D, BS = cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    print(f"reshape_and_cache_q8 cfg={cfg_id} decode={decode}", flush=True)
    if decode:
        ctx = np.array([1, BS, BS + 1, 3 * BS + 5, 2], np.int32)
        bt = gen.block_table(cfg, ctx)
        pos, seq, T = (ctx - 1).astype(np.int32), None, ctx.size
    else:
        pb = gen.packed([1, BS - 1, BS, BS + 1, 3 * BS + 5])
        bt = gen.block_table(cfg, pb.lens)
        pos, seq, T = pb.positions, pb.seq_of_token, pb.T
    bt.table[-1, pos[-1] // BS] = -1           # one invalid entry: its write is dropped
    k, v = rows_for(T, Hkv, D, dtype), rows_for(T, Hkv, D, dtype)
    empty = gen.empty_cache_q8(cfg, bt.num_blocks)
    dc = q8_dev(empty)
    dl.dl_reshape_and_cache(dev_as(k, dtype), dev_as(v, dtype),
                            dev_i32(seq) if seq is not None else None, dev_i32(pos),
                            dev_i32(bt.table), dc[0], dc[1], k_scale=dc[2], v_scale=dc[3])
    torch.cuda.synchronize()
    want = tuple(a.copy() for a in empty)
    sq = seq if seq is not None else np.arange(T, dtype=np.int32)
    keep = bt.table[sq, pos // BS] >= 0
    oracle.reshape_and_cache_q8(k[keep], v[keep], sq[keep], pos[keep], bt.table, *want)
    assert_q8_equal(q8_host(dc), want, f"cfg {cfg_id}")
    assert (want[0] != gen.CODE_SENTINEL).any()


DECODE_CASES = [  # B, ctx list, Hq, Hkv, D, BS
    (1, [1], 4, 4, 64, 16), (3, [5, 16, 17], 4, 4, 64, 16), (4, [130, 1, 700, 2049], 8, 1, 128, 128),
    (5, [127, 128, 129, 300, 64], 32, 8, 128, 128), (2, [4096, 3000], 8, 8, 128, 128),
    (3, [33, 64, 65], 8, 4, 64, 32),
]


def q8_decode_setup(B, ctx, Hq, Hkv, D, BS, dtype, identity=False):
    c = dataclasses.replace(gen.CONFIGS[4], n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                            block_size=BS, dtype="bf16" if dtype == torch.bfloat16 else "f32")
    bt = gen.block_table(c, ctx, identity=identity)
    cache = gen.synthetic_cache_q8(c, bt, np.asarray(ctx) + 1)   # fill positions 0..ctx-1
    return bt, cache


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,ctx,Hq,Hkv,D,BS", DECODE_CASES)
def test_attn_decode_paged_q8(dtype, B, ctx, Hq, Hkv, D, BS):
    print(f"attn_decode_q8 {dtype} ctx={ctx} {Hq}/{Hkv}x{D} BS={BS}", flush=True)
    bt, cache = q8_decode_setup(B, ctx, Hq, Hkv, D, BS, dtype)
    ctx = np.asarray(ctx, np.int32)
    q = R.standard_normal((B, Hq, D)).astype(np.float32)
    if dtype == torch.bfloat16:
        q = oracle.bf16_round(q)
    out = torch.empty(B, Hq, D, dtype=dtype, device=DEV)
    dc = q8_dev(cache)
    dl.dl_attn_decode_paged(dev_as(q, dtype), dc[0], dc[1], dev_i32(bt.table), dev_i32(ctx),
                            int(ctx.max()), out, k_scale=dc[2], v_scale=dc[3])
    mode = oracle.BF16 if dtype == torch.bfloat16 else oracle.EXACT
    ref = oracle.attn_decode_paged_q8(q, *cache, bt.table, ctx, mode=mode)
    if dtype == torch.bfloat16:
        assert_bf16_close(host(out), ref, "attn_decode_q8")
    else:
        assert_f32_close(host(out), ref, "attn_decode_q8", max_abs=1e-4, rel=1e-5)


def test_attn_decode_q8_permutation_bit_identical():
    ctx = np.array([513, 128, 1000, 7], np.int32)
    q = oracle.bf16_round(R.standard_normal((4, 32, 128)).astype(np.float32))
    outs = []
    for identity in (True, False):
        bt, cache = q8_decode_setup(4, ctx, 32, 8, 128, 128, torch.bfloat16, identity)
        dc = q8_dev(cache)
        out = torch.empty(4, 32, 128, dtype=torch.bfloat16, device=DEV)
        dl.dl_attn_decode_paged(dev_as(q, torch.bfloat16), dc[0], dc[1], dev_i32(bt.table),
                                dev_i32(ctx), int(ctx.max()), out, k_scale=dc[2], v_scale=dc[3])
        outs.append(host_bits(out))
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# whole layer with an INT8 cache
# ---------------------------------------------------------------------------

def small_gqa_cfg():
    return dataclasses.replace(gen.CONFIGS[4], config_id=41, name="gqa-small-q8", hidden=512,
                               n_q_heads=8, n_kv_heads=2, head_dim=128, intermediate=1408,
                               block_size=16)


def ws_kv(layer, ws, T, B, S_or_ctx, is_decode):
    """The layer's own k and v of its last call, read back from its
    workspace (the projection output the quantising cache write consumed)."""
    c = layer.cfg
    reg = dl.dl_layer_workspace_regions(layer.dims, T, B, S_or_ctx, is_decode, dl.DL_FUSED)
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    out = []
    for name in ("k", "v"):
        off, size = reg[name]
        out.append(host(ws[off:off + size].view(dt).view(T, c.n_kv_heads, c.head_dim)))
    return out


@pytest.mark.parametrize("cfg_name", ["tiny-f32", "gqa-bf16"])
def test_layer_q8_prefill_then_decode_vs_oracle(cfg_name):
    """The layer with an INT8 cache through a prefill and decode steps: every
    output against the oracle's INT8 layer, and after every call the cache
    equals, bit for bit, the oracle's quantising cache write applied to the
    k/v the GPU projection produced in that call (read back from the
    workspace), so no code is compared across different summation orders."""
    cfg = gen.CONFIGS[1] if cfg_name == "tiny-f32" else small_gqa_cfg()
    lens, steps = ([17, 1, 32], 3) if cfg_name == "tiny-f32" else ([100, 37, 300, 1], 3)
    print(f"layer q8 {cfg_name}", flush=True)
    pb = gen.packed(lens)
    x = gen.hidden(cfg, pb.T)
    bt = gen.block_table(cfg, pb.lens + steps)
    empty = gen.empty_cache_q8(cfg, bt.num_blocks)
    layer = DeviceLayer.build(cfg, max_pos=int(pb.lens.max()) + steps + 1, gamma="uniform")
    dc = q8_dev(empty)
    btd = i32(bt.table)
    oc = tuple(a.copy() for a in empty)        # the oracle's own chain
    mirror = tuple(a.copy() for a in empty)    # the oracle's write of the GPU's k/v
    omode = oracle.EXACT if cfg.dtype == "f32" else oracle.BF16
    close = (lambda g, r, w: assert_f32_close(g, r, w, max_abs=1e-3, rel=1e-5)) \
        if cfg.dtype == "f32" else (lambda g, r, w: assert_f32_close(g, r, w))
    d = cfg.dims()
    max_ctx = int(pb.lens.max()) + steps
    n = dl.dl_layer_workspace_size(layer.dims, pb.T, pb.B, pb.max_seqlen, max_ctx, dl.DL_FUSED)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    y = layer.prefill(to_dev(x, torch.float32), pb, dc[0], dc[1], btd, ws=ws, ks=dc[2],
                      vs=dc[3])
    torch.cuda.synchronize()
    y_ref, _ = oracle.layer_prefill_q8(d, layer.w_host, x, pb.positions, pb.seq_of_token,
                                       pb.cu_seqlens, *oc, bt.table, mode=omode)
    close(host(y), y_ref, f"{cfg_name} prefill")
    kg, vg = ws_kv(layer, ws, pb.T, pb.B, pb.max_seqlen, False)
    oracle.reshape_and_cache_q8(kg, vg, pb.seq_of_token, pb.positions, bt.table, *mirror)
    assert_q8_equal(q8_host(dc), mirror, f"{cfg_name} prefill cache")
    for s in range(steps):
        ctx = (pb.lens + s + 1).astype(np.int32)
        xd = gen.hidden(cfg, pb.B, step=100 + s)
        yd = layer.decode(to_dev(xd, torch.float32), ctx, dc[0], dc[1], btd, ws=ws, ks=dc[2],
                          vs=dc[3])
        torch.cuda.synchronize()
        yd_ref, _ = oracle.layer_decode_q8(d, layer.w_host, xd, ctx, *oc, bt.table, mode=omode)
        close(host(yd), yd_ref, f"{cfg_name} decode {s}")
        kg, vg = ws_kv(layer, ws, pb.B, pb.B, int(ctx.max()), True)
        oracle.reshape_and_cache_q8(kg, vg, np.arange(pb.B, dtype=np.int32), ctx - 1, bt.table,
                                    *mirror)
        assert_q8_equal(q8_host(dc), mirror, f"{cfg_name} decode {s} cache")
    got = q8_host(dc)
    written = oc[2] == oc[2]                    # rows whose oracle scale is not NaN
    assert np.array_equal(np.isnan(got[2]), ~written)   # the same rows were written
    for i in (0, 1):
        assert (got[i][~written] == gen.CODE_SENTINEL).all()


def test_layer_q8_fused_equals_step_by_step_bit_exact():
    cfg = small_gqa_cfg()
    pb = gen.packed([77, 130, 5])
    x = gen.hidden(cfg, pb.T)
    bt = gen.block_table(cfg, pb.lens + 2)
    empty = gen.empty_cache_q8(cfg, bt.num_blocks)
    layer = DeviceLayer.build(cfg, max_pos=200, gamma="uniform")
    xd = to_dev(x, torch.float32)
    c1, c2 = q8_dev(empty), q8_dev(empty)
    btd = i32(bt.table)
    y1 = layer.prefill(xd, pb, c1[0], c1[1], btd, ks=c1[2], vs=c1[3])
    s = layer.steps_prefill(xd, pb, c2[0], c2[1], btd, ks=c2[2], vs=c2[3])
    assert torch.equal(y1, s["y"])
    ctx = (pb.lens + 1).astype(np.int32)
    xdec = to_dev(gen.hidden(cfg, pb.B, step=7), torch.float32)
    yd1 = layer.decode(xdec, ctx, c1[0], c1[1], btd, ks=c1[2], vs=c1[3])
    sd = layer.steps_decode(xdec, ctx, c2[0], c2[1], btd, ks=c2[2], vs=c2[3])
    assert torch.equal(yd1, sd["y"])
    torch.cuda.synchronize()
    assert_q8_equal(q8_host(c1), q8_host(c2), "fused vs steps cache")


def test_layer_q8_unfused_mode_is_rejected():
    cfg = small_gqa_cfg()
    pb = gen.packed([8])
    bt = gen.block_table(cfg, pb.lens)
    dc = q8_dev(gen.empty_cache_q8(cfg, bt.num_blocks))
    layer = DeviceLayer.build(cfg, max_pos=16)
    with pytest.raises(dl.DLError, match="DL_FUSED"):
        layer.prefill(to_dev(gen.hidden(cfg, pb.T), torch.float32), pb, dc[0], dc[1],
                      i32(bt.table), mode=dl.DL_UNFUSED, ks=dc[2], vs=dc[3])
