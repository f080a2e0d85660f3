"""Parity at the full sizes of the five workload configurations, in the launch
configuration the benchmark times (one fused layer call per prefill or decode
step, workspace from dl_layer_workspace_size):

  * 7B prefill, B1 x 2048;
  * 7B decode, B64, contexts U{128..4096}, synthetic prior K/V;
  * 8B-GQA prefill of 8 ragged sequences U{256..1024}, then 128 decode steps
    on the cache that prefill wrote;
  * 70B decode, B4 x 4096 and B1 x 32768;
  * 7B decode B64 and 70B decode B1 x 32768 again with an INT8 KV cache.

The oracle cannot run these layers whole in seconds, so each step is checked
on sampled rows (every row where B is small): a sampled row is recomputed by
the oracle step from the GPU's own stored (bf16) inputs to that step, in the
oracle's bf16-storage mode.  Properties that hold at any size are checked in
full: the fused layer call equals the chain of exported step calls bit for
bit, the KV cache after the write equals the oracle's reshape-and-cache of
the GPU's k/v bit for bit (untouched slots keep their earlier bits), and
decode attention is compared for every (sequence, head).
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_decoder_layer_residual_amd import binding as dl
from transformer_decoder_layer_residual_amd import inputs as gen
from transformer_decoder_layer_residual_amd.harness import DeviceLayer, cache_dev, i32, to_dev

from _util import assert_bf16_close, assert_f32_close, bf16_ulp, host, host_bits, rel_l2

pytestmark = pytest.mark.gpu


def say(*a):
    print("[full-size]", *a, flush=True)


def sample_rows(T, n, seed, must=()):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.asarray(must, np.int64), r.integers(0, T, n)]))


def fused_ws(layer, T, B, max_seqlen, max_ctx):
    n = dl.dl_layer_workspace_size(layer.dims, T, B, max_seqlen, max_ctx, dl.DL_FUSED)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda:0")


def cache_bits_f32(bits):
    return np.ascontiguousarray(gen.cache_to_f32(bits))


def check_cache_write(got_dev, before_bits, k_gpu, v_gpu, seq, pos, table, which):
    """got_dev: the (K, V) device caches after the write; before_bits: their
    host bits before it.  The oracle writes the GPU's k/v into f32 copies."""
    ok = cache_bits_f32(before_bits[0])
    ov = cache_bits_f32(before_bits[1])
    oracle.reshape_and_cache(k_gpu, v_gpu, seq, pos, table, ok, ov)
    for got, want_f32 in ((got_dev[0], ok), (got_dev[1], ov)):
        want = gen.bf16_bits(want_f32)   # untouched NaN sentinels keep their payload bits
        g = host_bits(got)
        bad = g != want
        assert not bad.any(), f"{which}: {int(bad.sum())} cache elements differ from the oracle"
    return ok, ov


def check_tail(layer, s, x_host, rows, what):
    """O projection, residual + RMSNorm, gate/up + SiLU*mul and down + residual
    on the sampled rows, each from the GPU's own inputs to that step."""
    w, c = layer.w_host, layer.cfg
    T = x_host.shape[0]
    attn = host(s["attn"]).reshape(T, -1)[rows]
    o = host(s["o"])[rows]
    assert_bf16_close(o, oracle.linear(attn, w["wo"], round_bf16=True), f"{what} o")
    n2_ref, h_ref = oracle.rmsnorm(o, w["ln2"], c.rms_eps, resid=x_host[rows], mode=oracle.BF16)
    assert_f32_close(host(s["h"])[rows], h_ref, f"{what} h", max_abs=1e-5, rel=1e-6)
    n2 = host(s["n2"])[rows]
    assert_bf16_close(n2, n2_ref, f"{what} n2")
    a = host(s["a"])[rows]
    assert_bf16_close(a, oracle.swiglu(n2, w["wg"], w["wu"], mode=oracle.BF16), f"{what} a")
    y_ref = oracle.down_residual(a, w["wd"], host(s["h"])[rows])
    assert_f32_close(host(s["y"])[rows], y_ref, f"{what} y")


def check_head(layer, s, x_host, pos, rows, what):
    """Input RMSNorm and the QKV + RoPE projection on the sampled rows."""
    w, c = layer.w_host, layer.cfg
    n1 = host(s["n1"])[rows]
    assert_bf16_close(n1, oracle.rmsnorm(x_host[rows], w["ln1"], c.rms_eps, mode=oracle.BF16),
                      f"{what} n1")
    rq, rk, rv = oracle.qkv_rope(n1, w["wq"], w["wk"], w["wv"], pos[rows], c.rope_theta,
                                 c.n_q_heads, c.n_kv_heads, c.head_dim, mode=oracle.BF16)
    assert_bf16_close(host(s["q"])[rows], rq, f"{what} q")
    assert_bf16_close(host(s["k"])[rows], rk, f"{what} k")
    assert_bf16_close(host(s["v"])[rows], rv, f"{what} v")


def check_prefill_attention(s, pb, rows, what):
    """Causal attention of the sampled query rows over their own sequence's
    keys 0..p, as single-query attention over a contiguous copy of those
    keys (the same softmax over the same visible set)."""
    q, k, v = host(s["q"]), host(s["k"]), host(s["v"])
    Hkv, D = k.shape[1], k.shape[2]
    ctx = (pb.positions[rows] + 1).astype(np.int32)
    S = int(ctx.max())
    kc = np.zeros((rows.size, Hkv, S, D), np.float32)
    vc = np.zeros_like(kc)
    for i, t in enumerate(rows):
        start = int(pb.cu_seqlens[pb.seq_of_token[t]])
        n = int(ctx[i])
        kc[i, :, :n] = k[start:start + n].transpose(1, 0, 2)
        vc[i, :, :n] = v[start:start + n].transpose(1, 0, 2)
    ref = oracle.attn_decode_contig(q[rows], kc, vc, ctx, mode=oracle.BF16)
    assert_bf16_close(host(s["attn"])[rows], ref, f"{what} attn")


# ---------------------------------------------------------------------------
# prefill: 7B B1 x 2048 and 8B-GQA ragged B8 (then its 128 decode steps)
# ---------------------------------------------------------------------------

def run_full_prefill(cfg, decode_capacity=0):
    pb = gen.prefill_batch(cfg)
    say(f"{cfg.name}: T={pb.T} B={pb.B} lens {pb.lens.min()}..{pb.lens.max()}")
    layer = DeviceLayer.build(cfg, max_pos=int(pb.lens.max()) + decode_capacity + 1)
    x = gen.hidden(cfg, pb.T)
    bt = gen.block_table(cfg, pb.lens + decode_capacity)
    kb, vb = gen.empty_cache(cfg, bt.num_blocks)
    kc1, vc1, kc2, vc2 = cache_dev(kb), cache_dev(vb), cache_dev(kb), cache_dev(vb)
    btd = i32(bt.table)
    xd = to_dev(x, torch.float32)
    ws = fused_ws(layer, pb.T, pb.B, pb.max_seqlen, 0)
    y = layer.prefill(xd, pb, kc1, vc1, btd, ws=ws)
    s = layer.steps_prefill(xd, pb, kc2, vc2, btd)
    torch.cuda.synchronize()
    assert torch.equal(y, s["y"]), "fused prefill differs from the step-by-step chain"
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))
    starts = pb.cu_seqlens[:-1]
    rows = sample_rows(pb.T, 10, cfg.config_id, must=[0, pb.T - 1, *starts[:2], *(starts[1:3] - 1)])
    say(f"{cfg.name}: sampled rows {rows.tolist()}")
    check_head(layer, s, x, pb.positions, rows, cfg.name)
    check_cache_write((kc1, vc1), (kb, vb), host(s["k"]), host(s["v"]), pb.seq_of_token,
                      pb.positions, bt.table, f"{cfg.name} cache")
    check_prefill_attention(s, pb, rows, cfg.name)
    check_tail(layer, s, x, rows, cfg.name)
    return layer, pb, bt, (kc1, vc1), btd, xd, y


def assert_probs_close(gpu, ref, what):
    """Softmax probabilities stored in bf16 by both sides: each within one
    bf16 ulp of the oracle's (the scores they come from differ only by fp32
    summation order, so at most one rounding boundary flips)."""
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    assert np.isfinite(gpu).all(), f"{what}: non-finite probabilities"
    bound = np.maximum(bf16_ulp(ref), np.float32(1e-30))
    bad = np.abs(gpu - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} probabilities beyond one bf16 ulp"
    assert rel_l2(gpu, ref) <= 1e-2, what


def check_unfused_chain(layer, pb, bt, btd, xd, x_host, y_fused, rows, what):
    """The kernel-per-op chain at full size, every stored intermediate read
    back from the layer workspace (dl_layer_workspace_regions) and compared
    element by element on the sampled rows with the oracle's BF16_UNFUSED
    steps, each fed the GPU's own inputs to that step: n1; q, k (rounded
    before and after RoPE) and v; the fp32 score rows and the bf16
    probability rows of every head (masked keys -inf / 0); the attention
    output; o; h; n2; gate, up, silu(gate) and a; the fp32 down projection;
    y.  The cache it writes is the oracle's reshape-and-cache of its own k/v
    bit for bit."""
    c, w = layer.cfg, layer.w_host
    T, B, S = pb.T, pb.B, pb.max_seqlen
    H, Hq, Hkv, D, I = c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.intermediate
    dt = torch.bfloat16
    n = dl.dl_layer_workspace_size(layer.dims, T, B, S, 0, dl.DL_UNFUSED)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    kb, vb = gen.empty_cache(c, bt.num_blocks)
    kc, vc = cache_dev(kb), cache_dev(vb)
    yu = layer.prefill(xd, pb, kc, vc, btd, mode=dl.DL_UNFUSED, ws=ws)
    torch.cuda.synchronize()
    reg = dl.dl_layer_workspace_regions(layer.dims, T, B, S, False, dl.DL_UNFUSED)

    def region(name, dtype, shape):
        off, size = reg[name]
        assert size == int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size(), name
        return ws[off:off + size].view(dtype).view(*shape)

    n1 = host(region("n1", dt, (T, H)))[rows]
    assert_bf16_close(n1, oracle.rmsnorm(x_host[rows], w["ln1"], c.rms_eps, mode=oracle.BF16),
                      f"{what} unfused n1")
    q_all = host(region("q", dt, (T, Hq, D)))
    k_all = host(region("k", dt, (T, Hkv, D)))
    v_all = host(region("v", dt, (T, Hkv, D)))
    rq, rk, rv = oracle.qkv_rope(n1, w["wq"], w["wk"], w["wv"], pb.positions[rows], c.rope_theta,
                                 Hq, Hkv, D, mode=oracle.BF16_UNFUSED)
    assert_bf16_close(q_all[rows], rq, f"{what} unfused q")
    assert_bf16_close(k_all[rows], rk, f"{what} unfused k")
    assert_bf16_close(v_all[rows], rv, f"{what} unfused v")
    check_cache_write((kc, vc), (kb, vb), k_all, v_all, pb.seq_of_token, pb.positions, bt.table,
                      f"{what} unfused cache")
    scores = region("scores", torch.float32, (B, Hq, S, S))
    probs = region("probs", dt, (B, Hq, S, S))
    attn = host(region("attn", dt, (T, Hq * D)))[rows].reshape(-1, Hq, D)
    G = Hq // Hkv
    for r_i, t in enumerate(rows):
        b = int(pb.seq_of_token[t])
        t0 = int(pb.cu_seqlens[b])
        Sb = int(pb.cu_seqlens[b + 1]) - t0
        i = int(t) - t0
        s_row = host(scores[b, :, i, :Sb])
        p_row = host(probs[b, :, i, :Sb])
        assert np.all(np.isneginf(s_row[:, i + 1:])), f"{what} row {t}: unmasked scores"
        assert np.all(p_row[:, i + 1:] == 0), f"{what} row {t}: probabilities past the diagonal"
        o_ref = np.empty((Hq, D), np.float32)
        for h in range(Hq):
            g = h // G
            s_ref, p_ref, o_ref[h] = oracle.attn_row(q_all[t, h], k_all[t0:t0 + i + 1, g],
                                                     v_all[t0:t0 + i + 1, g],
                                                     mode=oracle.BF16_UNFUSED)
            assert_f32_close(s_row[h, :i + 1], s_ref, f"{what} row {t} head {h} scores",
                             max_abs=1e-3, rel=1e-5)
            assert_probs_close(p_row[h, :i + 1], p_ref, f"{what} row {t} head {h} probs")
        assert_bf16_close(attn[r_i], o_ref, f"{what} row {t} unfused attn")
    attn = attn.reshape(len(rows), Hq * D)
    o = host(region("o", dt, (T, H)))[rows]
    assert_bf16_close(o, oracle.linear(attn, w["wo"], round_bf16=True), f"{what} unfused o")
    h = host(region("h", torch.float32, (T, H)))[rows]
    n2_ref, h_ref = oracle.rmsnorm(o, w["ln2"], c.rms_eps, resid=x_host[rows], mode=oracle.BF16)
    assert np.array_equal(h, h_ref), f"{what} unfused h: the fp32 residual add is exact"
    n2 = host(region("n2", dt, (T, H)))[rows]
    assert_bf16_close(n2, n2_ref, f"{what} unfused n2")
    g_ref, u_ref, sg_ref, a_ref = oracle.swiglu_parts(n2, w["wg"], w["wu"],
                                                      mode=oracle.BF16_UNFUSED)
    for name, ref in (("gate", g_ref), ("up", u_ref), ("silu", sg_ref), ("a", a_ref)):
        assert_bf16_close(host(region(name, dt, (T, I)))[rows], ref, f"{what} unfused {name}")
    a = host(region("a", dt, (T, I)))[rows]
    dd = host(region("down", torch.float32, (T, H)))[rows]
    assert_f32_close(dd, oracle.down_residual(a, w["wd"]), f"{what} unfused down")
    yr = host(yu)[rows]
    assert np.array_equal(yr, (h + dd).astype(np.float32)), f"{what} unfused y = h + down"
    assert_f32_close(yr, oracle.down_residual(a, w["wd"], h), f"{what} unfused y")
    # the two modes round at different places; reported, not gated
    r = rel_l2(host(yu), host(y_fused))
    say(f"{what}: fused vs unfused rel-L2 {r:.2e}, max-abs {float((yu - y_fused).abs().max()):.3e}")


def test_llama2_7b_prefill_full_size():
    cfg = gen.CONFIGS[2]
    layer, pb, bt, caches, btd, xd, y = run_full_prefill(cfg)
    rows = sample_rows(pb.T, 10, 21, must=[0, 1, 127, 128, pb.T - 1])
    check_unfused_chain(layer, pb, bt, btd, xd, gen.hidden(cfg, pb.T), y, rows, cfg.name)


def decode_step_checked(layer, x_host, ctx, caches, bt, btd, what, rows=None):
    """One fused decode step on `caches` (updated in place) and the same step
    through the exported calls on a copy; both compared, then sampled rows
    and every attention output against the oracle."""
    c = layer.cfg
    B = x_host.shape[0]
    kb, vb = host_bits(caches[0]), host_bits(caches[1])
    kc2, vc2 = caches[0].clone(), caches[1].clone()
    xd = to_dev(x_host, torch.float32)
    ws = fused_ws(layer, B, B, 0, int(ctx.max()))
    y = layer.decode(xd, ctx, caches[0], caches[1], btd, ws=ws)
    s = layer.steps_decode(xd, ctx, kc2, vc2, btd)
    torch.cuda.synchronize()
    assert torch.equal(y, s["y"]), f"{what}: fused decode differs from the step-by-step chain"
    assert torch.equal(caches[0].view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(caches[1].view(torch.int16), vc2.view(torch.int16))
    del kc2, vc2
    pos = (ctx - 1).astype(np.int32)
    rows = np.arange(B) if rows is None else rows
    check_head(layer, s, x_host, pos, rows, what)
    ok, ov = check_cache_write(caches, (kb, vb), host(s["k"]), host(s["v"]),
                               np.arange(B, dtype=np.int32), pos, bt.table, f"{what} cache")
    del kb, vb
    ref = oracle.attn_decode_paged(host(s["q"]), ok, ov, bt.table, ctx, mode=oracle.BF16)
    del ok, ov
    assert_bf16_close(host(s["attn"]), ref, f"{what} attn")
    check_tail(layer, s, x_host, rows, what)
    return y


def test_llama3_8b_gqa_prefill_then_128_decode_steps():
    cfg = gen.CONFIGS[4]
    layer, pb, bt, caches, btd, xd, y = run_full_prefill(cfg, decode_capacity=cfg.decode_steps)
    starts = pb.cu_seqlens[:-1]
    rows = sample_rows(pb.T, 6, 41, must=[0, pb.T - 1, *starts[1:3], *(starts[1:3] - 1)])
    check_unfused_chain(layer, pb, bt, btd, xd, gen.hidden(cfg, pb.T), y, rows, cfg.name)
    checked = {0, cfg.decode_steps // 2, cfg.decode_steps - 1}
    for step in range(cfg.decode_steps):
        ctx = (pb.lens + step + 1).astype(np.int32)
        x = gen.hidden(cfg, pb.B, step=1 + step)
        if step in checked:
            say(f"{cfg.name}: decode step {step}, ctx {ctx.min()}..{ctx.max()}")
            decode_step_checked(layer, x, ctx, caches, bt, btd, f"{cfg.name} decode {step}")
        else:
            layer.decode(to_dev(x, torch.float32), ctx, caches[0], caches[1], btd)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# decode without a prefill of its own: 7B B64, 70B B4 x 4096 and B1 x 32768
# ---------------------------------------------------------------------------

def run_full_decode(layer, ctx, case, rows=None):
    cfg = layer.cfg
    bt = gen.block_table(cfg, ctx)
    kb, vb = gen.synthetic_cache(cfg, bt, ctx, case=case)
    caches = (cache_dev(kb), cache_dev(vb))
    del kb, vb
    x = gen.hidden(cfg, ctx.size, step=1 + case)
    say(f"{cfg.name}: B={ctx.size} ctx {ctx.min()}..{ctx.max()} ({bt.num_blocks} blocks)")
    decode_step_checked(layer, x, ctx, caches, bt, i32(bt.table), f"{cfg.name} case {case}",
                        rows=rows)


def test_llama2_7b_decode_full_size():
    cfg = gen.CONFIGS[3]
    ctx = gen.decode_context_lens(cfg)
    layer = DeviceLayer.build(cfg, max_pos=int(ctx.max()) + 1)
    run_full_decode(layer, ctx, 0, rows=sample_rows(ctx.size, 12, 3, must=[0, ctx.size - 1]))


@pytest.fixture(scope="module")
def layer_70b():
    cfg = gen.CONFIGS[5]
    say(f"{cfg.name}: building weights")
    return DeviceLayer.build(cfg, max_pos=max(c for _, c in cfg.extra["cases"]) + 1)


@pytest.mark.parametrize("case", [0, 1])
def test_llama_70b_decode_full_size(layer_70b, case):
    run_full_decode(layer_70b, gen.decode_context_lens(layer_70b.cfg, case), case)


# ---------------------------------------------------------------------------
# INT8 KV cache at full size
# ---------------------------------------------------------------------------

def q8_equal(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def decode_step_checked_q8(layer, x_host, ctx, caches, bt, btd, what, rows=None):
    """decode_step_checked for an INT8 cache (codes k, v and scales k, v):
    fused equals step by step bit for bit, the cache write is the oracle's
    quantisation of the GPU's own k/v bit for bit, and every (sequence, head)
    of attention matches the oracle's INT8 attention over that cache."""
    B = x_host.shape[0]
    before = tuple(t.cpu().numpy() for t in caches)
    c2 = tuple(t.clone() for t in caches)
    xd = to_dev(x_host, torch.float32)
    ws = fused_ws(layer, B, B, 0, int(ctx.max()))
    y = layer.decode(xd, ctx, caches[0], caches[1], btd, ws=ws, ks=caches[2], vs=caches[3])
    s = layer.steps_decode(xd, ctx, c2[0], c2[1], btd, ks=c2[2], vs=c2[3])
    torch.cuda.synchronize()
    assert torch.equal(y, s["y"]), f"{what}: fused decode differs from the step-by-step chain"
    assert all(q8_equal(a, b) for a, b in zip(caches, c2)), f"{what}: caches differ"
    del c2
    pos = (ctx - 1).astype(np.int32)
    rows = np.arange(B) if rows is None else rows
    check_head(layer, s, x_host, pos, rows, what)
    want = tuple(a.copy() for a in before)
    del before
    oracle.reshape_and_cache_q8(host(s["k"]), host(s["v"]), np.arange(B, dtype=np.int32), pos,
                                bt.table, *want)
    for got, w, name in zip(caches, want, ("k codes", "v codes", "k scales", "v scales")):
        g = got.cpu().numpy()
        same = (g.view(np.uint32) == w.view(np.uint32)) if g.dtype == np.float32 else (g == w)
        assert same.all(), f"{what}: {int((~same).sum())} {name} differ from the oracle"
    ref = oracle.attn_decode_paged_q8(host(s["q"]), *want, bt.table, ctx, mode=oracle.BF16)
    del want
    assert_bf16_close(host(s["attn"]), ref, f"{what} attn")
    check_tail(layer, s, x_host, rows, what)
    return y


def run_full_decode_q8(layer, ctx, case, rows=None):
    cfg = layer.cfg
    bt = gen.block_table(cfg, ctx)
    caches = tuple(cache_dev(a) for a in gen.synthetic_cache_q8(cfg, bt, ctx, case=case))
    x = gen.hidden(cfg, ctx.size, step=1 + case)
    say(f"{cfg.name} INT8 cache: B={ctx.size} ctx {ctx.min()}..{ctx.max()} "
        f"({bt.num_blocks} blocks)")
    decode_step_checked_q8(layer, x, ctx, caches, bt, i32(bt.table),
                           f"{cfg.name} int8 case {case}", rows=rows)


def test_llama2_7b_decode_int8_cache_full_size():
    cfg = gen.CONFIGS[3]
    ctx = gen.decode_context_lens(cfg)
    layer = DeviceLayer.build(cfg, max_pos=int(ctx.max()) + 1)
    run_full_decode_q8(layer, ctx, 0, rows=sample_rows(ctx.size, 12, 5, must=[0, ctx.size - 1]))


def test_llama_70b_decode_int8_cache_full_size(layer_70b):
    run_full_decode_q8(layer_70b, gen.decode_context_lens(layer_70b.cfg, 1), 1)
