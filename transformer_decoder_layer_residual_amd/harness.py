"""Device-side setup of a whole decoder layer (tests, smoke check and bench).

Builds the weights, RoPE table, paged caches and block table of a workload
configuration on the GPU (all values from the seeded generator) and runs the
layer through the C ABI, either fused (one call) or step by step (one call
per exported step, the same kernels in the same order).
"""
import dataclasses

import numpy as np
import torch

from . import binding as dl
from . import inputs as gen

DEV = "cuda:0"


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    return t.to(dtype) if dtype != torch.float32 else t


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def cache_dev(bits):
    """Host cache -> device: bf16 / fp32 bit patterns, int8 codes or fp32 scales."""
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    if bits.dtype == np.int8:
        return torch.from_numpy(np.ascontiguousarray(bits)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).to(DEV)


@dataclasses.dataclass
class DeviceLayer:
    cfg: object
    w_host: dict
    w: dict
    dims: object
    cs: torch.Tensor
    max_pos: int

    @classmethod
    def build(cls, cfg, max_pos, gamma="ones", w_host=None):
        dt = torch_dtype(cfg)
        w_host = gen.weights(cfg, gamma=gamma) if w_host is None else w_host
        w = {k: to_dev(v, dt) for k, v in w_host.items()}
        dims = dl.make_dims(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                            cfg.intermediate, cfg.block_size, cfg.rms_eps, dt)
        cs = torch.empty(max_pos, cfg.head_dim, device=DEV)
        dl.dl_rope_table_fill(cs, max_pos, cfg.head_dim, cfg.rope_theta)
        return cls(cfg, w_host, w, dims, cs, max_pos)

    # -- fused (ks, vs: row scales of an int8 cache) -------------------------
    def prefill(self, x, pb, kc, vc, bt_dev, mode=dl.DL_FUSED, ws=None, ks=None, vs=None):
        y = torch.empty_like(x)
        dl.dl_layer_prefill(self.dims, self.w, self.cs, x, y, i32(pb.positions),
                            i32(pb.seq_of_token), i32(pb.cu_seqlens), pb.max_seqlen, kc, vc,
                            bt_dev, mode=mode, ws=ws, k_scale=ks, v_scale=vs)
        return y

    def decode(self, x, ctx, kc, vc, bt_dev, mode=dl.DL_FUSED, ws=None, ks=None, vs=None):
        y = torch.empty_like(x)
        ctx = np.asarray(ctx, np.int32)
        dl.dl_layer_decode(self.dims, self.w, self.cs, x, y, i32(ctx - 1), i32(ctx),
                           int(ctx.max()), kc, vc, bt_dev, mode=mode, ws=ws, k_scale=ks,
                           v_scale=vs)
        return y

    def decode_qlens(self, x, qb, ctx, kc, vc, bt_dev, ws=None):
        """New tokens appended to cached sequences: qb is the packed batch of
        the new tokens (lens = q_len per sequence), ctx the context lengths
        after the step."""
        y = torch.empty_like(x)
        ctx = np.asarray(ctx, np.int32)
        pos = (np.repeat(ctx - qb.lens, qb.lens) + qb.positions).astype(np.int32)
        dl.dl_layer_decode_qlens(self.dims, self.w, self.cs, x, y, i32(pos), i32(qb.seq_of_token),
                                 i32(qb.cu_seqlens), i32(ctx), qb.max_seqlen, int(ctx.max()), kc,
                                 vc, bt_dev, ws=ws)
        return y

    # -- step by step (exported step entry points) ---------------------------
    def steps_prefill(self, x, pb, kc, vc, bt_dev, gu_events=None, ks=None, vs=None):
        c, dt = self.cfg, torch_dtype(self.cfg)
        T, H, Hq, Hkv, D, I = pb.T, c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.intermediate
        s = {}
        s["n1"] = torch.empty(T, H, dtype=dt, device=DEV)
        dl.dl_rmsnorm_residual(x, self.w["ln1"], s["n1"], c.rms_eps)
        s["q"] = torch.empty(T, Hq, D, dtype=dt, device=DEV)
        s["k"] = torch.empty(T, Hkv, D, dtype=dt, device=DEV)
        s["v"] = torch.empty(T, Hkv, D, dtype=dt, device=DEV)
        pos = i32(pb.positions)
        dl.dl_qkv_rope(s["n1"], self.w["wq"], self.w["wk"], self.w["wv"], pos, self.cs, s["q"],
                       s["k"], s["v"])
        dl.dl_reshape_and_cache(s["k"], s["v"], i32(pb.seq_of_token), pos, bt_dev, kc, vc,
                                k_scale=ks, v_scale=vs)
        s["attn"] = torch.empty(T, Hq, D, dtype=dt, device=DEV)
        dl.dl_attn_prefill(s["q"], s["k"], s["v"], i32(pb.cu_seqlens), pb.max_seqlen, s["attn"])
        return self._tail(x, s, T, H, I, dt, gu_events)

    def steps_decode(self, x, ctx, kc, vc, bt_dev, ks=None, vs=None):
        c, dt = self.cfg, torch_dtype(self.cfg)
        B, H, Hq, Hkv, D, I = x.shape[0], c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, \
            c.intermediate
        ctx = np.asarray(ctx, np.int32)
        s = {}
        s["n1"] = torch.empty(B, H, dtype=dt, device=DEV)
        dl.dl_rmsnorm_residual(x, self.w["ln1"], s["n1"], c.rms_eps)
        s["q"] = torch.empty(B, Hq, D, dtype=dt, device=DEV)
        s["k"] = torch.empty(B, Hkv, D, dtype=dt, device=DEV)
        s["v"] = torch.empty(B, Hkv, D, dtype=dt, device=DEV)
        pos = i32(ctx - 1)
        dl.dl_qkv_rope(s["n1"], self.w["wq"], self.w["wk"], self.w["wv"], pos, self.cs, s["q"],
                       s["k"], s["v"])
        dl.dl_reshape_and_cache(s["k"], s["v"], None, pos, bt_dev, kc, vc, k_scale=ks, v_scale=vs)
        s["attn"] = torch.empty(B, Hq, D, dtype=dt, device=DEV)
        dl.dl_attn_decode_paged(s["q"], kc, vc, bt_dev, i32(ctx), int(ctx.max()), s["attn"],
                                k_scale=ks, v_scale=vs)
        return self._tail(x, s, B, H, I, dt)

    def _tail(self, x, s, T, H, I, dt, gu_events=None):
        c = self.cfg
        s["o"] = torch.empty(T, H, dtype=dt, device=DEV)
        dl.dl_linear(s["attn"].view(T, -1), self.w["wo"], s["o"])
        s["n2"] = torch.empty(T, H, dtype=dt, device=DEV)
        s["h"] = torch.empty(T, H, device=DEV)
        dl.dl_rmsnorm_residual(s["o"], self.w["ln2"], s["n2"], c.rms_eps, residual_in=x,
                               residual_out=s["h"])
        s["a"] = torch.empty(T, I, dtype=dt, device=DEV)
        ws = None
        if gu_events is not None:   # time the gate/up launch alone, inside the chain
            n = dl.lib().dl_gate_up_silu_workspace_size(T, H, I, dl.dtype_code(dt))
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
            gu_events[0].record()
        dl.dl_gate_up_silu(s["n2"], self.w["wg"], self.w["wu"], s["a"], ws=ws)
        if gu_events is not None:
            gu_events[1].record()
        s["y"] = torch.empty(T, H, device=DEV)
        dl.dl_down_residual(s["a"], self.w["wd"], s["y"], residual=s["h"])
        return s


def prefill_inputs(cfg, pb, extra_capacity=0, identity=False):
    """x, block table and sentinel caches for a prefill of batch pb."""
    x = gen.hidden(cfg, pb.T)
    bt = gen.block_table(cfg, pb.lens + extra_capacity, identity=identity)
    kbits, vbits = gen.empty_cache(cfg, bt.num_blocks)
    return x, bt, kbits, vbits
