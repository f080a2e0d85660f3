#!/usr/bin/env python
"""Decoder-layer benchmark on one MI355X.

Step = one dl_layer_prefill call on the Llama-2-7B-shaped layer (hidden 4096,
32 heads x 128, intermediate 11008, bf16) over one 2048-token sequence: input
RMSNorm, merged QKV GEMM + RoPE, reshape-and-cache, causal flash attention,
O-projection, RMSNorm fused with the residual add, gate/up GEMM + SiLU*mul,
down GEMM + residual.  value = prefill tokens/s of the layer.

Beside it the JSON line carries:
  roofline      the gate/up GEMM (the layer's largest kernel), timed with HIP
                events around its launches inside the step-by-step layer chain,
                on the stream it is launched on, against bf16 MFMA peak;
  layer         whole-step flops and the fraction of peak;
  decode        one decode step of the same layer shape at batch 64 with
                context lengths U{128..4096} over a paged cache (tokens/s and
                the paged attention kernel against HBM peak);
  decode_kv_int8  the same decode step over an INT8 KV cache with per-token
                scales (quantised on write, dequantised by the attention);
  verify_qlen4  the same batch verifying 4 candidate tokens per sequence in
                one layer step (paged attention with per-sequence q_len);
  decode_small_batch  the Llama-3-8B-shaped layer at B8, eager calls against
                the step replayed as one HIP graph, back to back and with a
                host synchronisation after every step (decode lines above also
                carry their graph timing);
  prefill_gqa_8b  the Llama-3-8B-shaped GQA layer prefilling 8 ragged
                sequences U{256..1024} (tokens/s, its gate/up GEMM roofline);
  cpu_baseline  the CPU oracle on a bounded prefix of the same prefill (all
                host threads; the decode and tiny-layer samples also on one).

Inputs are resident in HBM before the timed region; weights and activations
are seeded synthetic data.  Timed steps are cold: before every step, outside
its HIP event pair, a 1 GiB buffer is written (evicting the L2s and the 256 MB
MALL) and another 1 GiB read (draining the write-backs), and the step's time
is the median over the steps; back-to-back (warm) means are reported beside
them.  Every timed line names its
cache_state.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decoder-layer tokens/s (prefill, decode) + % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
SPEC_CLOCK_MHZ = 2400.0        # clock the published peaks are quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic.json), used only if it was taken on the current kernel
    source; else None."""
    from transformer_decoder_layer_residual_amd import profiling
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel_key)
    except (OSError, ValueError):
        return None
    srcs = profiling.KERNELS[kernel_key][1]
    if not rec or rec.get("source_sha") != profiling.source_sha(*srcs):
        return None
    return rec.get("bytes_per_launch")


def gfx_clock_mhz():
    """Current graphics clock from `amd-smi metric -c --json` (a child
    process), averaged over the GPU's XCD clock domains; with several GPUs
    listed, the busiest (highest) one.  None when the tool is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True,
                           text=True, timeout=30)
        d = json.loads(r.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    gpus = d.get("gpu_data", []) if isinstance(d, dict) else d
    best = None
    for g in gpus if isinstance(gpus, list) else []:
        vals = []
        for k, v in (g.get("clock") or {}).items():
            c = v.get("clk") if isinstance(v, dict) and k.startswith("gfx") else None
            if isinstance(c, dict) and isinstance(c.get("value"), (int, float)):
                vals.append(float(c["value"]))
        if vals:
            m = sum(vals) / len(vals)
            best = m if best is None else max(best, m)
    return best


class ClockSampler:
    """Graphics-clock readings from a child process started before this
    process touches the GPU (the child runs amd-smi every half second and
    prints time-stamped readings; nothing is started from the GPU process).
    under(fn) keeps fn repeating on the GPU for a few seconds and averages the
    readings taken in that window, skipping its first 2 s (the reported
    clock lags the load by about a second)."""

    def __init__(self):
        import subprocess
        import threading
        self.samples = []
        self.proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--clock-sampler"],
                                     stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)

        def reader():
            for line in self.proc.stdout:
                t, _, v = line.strip().partition(" ")
                try:
                    self.samples.append((float(t), float(v)))
                except ValueError:
                    pass

        self.th = threading.Thread(target=reader, daemon=True)
        self.th.start()

    def under(self, fn, stream, seconds=4.5):
        t0 = time.time()
        while time.time() - t0 < seconds:
            for _ in range(10):
                fn()
            stream.synchronize()
        t1 = time.time()
        time.sleep(0.6)                       # the reading of the window's last moments
        vals = [v for t, v in self.samples if t0 + 2.0 <= t <= t1]
        return round(sum(vals) / len(vals), 1) if vals else None

    def close(self):
        if self.proc.poll() is None:
            self.proc.terminate()
            try:
                self.proc.wait(timeout=10)
            except Exception:
                self.proc.kill()


class NoClock:
    """Stands in for ClockSampler when no child may be started."""

    def under(self, fn, stream, seconds=0.0):
        return None

    def close(self):
        pass


def clock_sampler_child(limit_s=1200.0):
    """The sampler child's loop (never initialises the GPU)."""
    t0 = time.time()
    while time.time() - t0 < limit_s:
        v = gfx_clock_mhz()
        print(f"{time.time():.3f} {v if v is not None else 'none'}", flush=True)
        if v is None:
            return
        time.sleep(0.5)


def time_synced(fn, n, stream):
    """Wall time of n steps that each end with a host synchronisation (the
    serving-loop pattern, where host launch latency is not hidden)."""
    stream.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
        stream.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n


FLUSH_BYTES = 1 << 30


class Flusher:
    """Writes a 1 GiB device buffer (a fill kernel on the timing stream), which
    evicts every L2 and the MALL between timed steps, then reads another 1 GiB
    buffer (a sum), so the write-backs of the written lines drain before the
    timed step instead of competing with its reads (with the write alone,
    the 70B-shaped decode gate/up measured 217 us against 155 us)."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
        self.rbuf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
        self.acc = None
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k)
        self.acc = self.rbuf.sum()


def time_cold(fn, n, stream, flush):
    """n steps, each preceded by a cache flush outside its event pair: (median,
    p10, p90) in ms."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: t[min(len(t) - 1, int(f * len(t)))]
    return t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2]), \
        q(0.1), q(0.9)


def warm_up(fn, n, stream, min_s=1.0):
    """At least n steps and at least min_s seconds of them (the clocks settle
    under sustained load)."""
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < min_s:
        fn()
        i += 1
        if i % 8 == 0:
            stream.synchronize()
    stream.synchronize()


def time_launches(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n   # ms per launch


def host_cpu():
    """CPU model, sockets and logical CPUs of the host (lscpu)."""
    import subprocess
    info = {"logical_cpus": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    for line in out.splitlines():
        k, _, v = line.partition(":")
        k, v = k.strip(), v.strip()
        if k == "Model name":
            info["model"] = v
        elif k == "Socket(s)":
            info["sockets"] = int(v) if v.isdigit() else v
        elif k == "Core(s) per socket":
            info["cores_per_socket"] = int(v) if v.isdigit() else v
    return info


def cpu_sample(kind: str, ready=None) -> dict:
    """A bounded CPU-oracle sample (no GPU): 'tiny' = the tiny fp32 layer's
    32-token prefill then 8 decode steps on its own cache; 'decode' = the 7B
    decode layer step for the first 4 sequences of the 7B decode workload.
    `ready`, if given, is called once the inputs are built and returns when
    the timed part may start."""
    import numpy as np

    import oracle
    from transformer_decoder_layer_residual_amd import inputs as gen
    if kind == "tiny":
        cfg = gen.CONFIGS[1]
        w = gen.weights(cfg)
        pb = gen.prefill_batch(cfg)
        bt = gen.block_table(cfg, pb.lens + cfg.decode_steps)
        kb, vb = gen.empty_cache(cfg, bt.num_blocks)
        kf, vf = gen.cache_to_f32(kb).copy(), gen.cache_to_f32(vb).copy()
        x = gen.hidden(cfg, pb.T)
        xs = [gen.hidden(cfg, 1, step=1 + s) for s in range(cfg.decode_steps)]
        if ready:
            ready()

        def one_pass():
            # the cache is rewritten in place each pass (same values)
            t0 = time.perf_counter()
            oracle.layer_prefill(cfg.dims(), w, x, pb.positions, pb.seq_of_token, pb.cu_seqlens,
                                 kf, vf, bt.table, mode=oracle.EXACT)
            t1 = time.perf_counter()
            for s in range(cfg.decode_steps):
                ctx = np.array([pb.T + s + 1], np.int32)
                oracle.layer_decode(cfg.dims(), w, xs[s], ctx, kf, vf, bt.table,
                                    mode=oracle.EXACT)
            return t1 - t0, time.perf_counter() - t1

        one_pass()                             # first-call costs (thread pool, page faults)
        reps = 5
        tp = td = 0.0
        for _ in range(reps):
            a, b = one_pass()
            tp += a
            td += b
        return {"prefill_tokens_per_s": round(reps * pb.T / tp, 1),
                "decode_tokens_per_s": round(reps * cfg.decode_steps / td, 1),
                "seconds": round(tp + td, 4), "passes": reps}
    cfg = gen.CONFIGS[3]
    nb = 4
    w = gen.weights(cfg)
    ctx = gen.decode_context_lens(cfg)[:nb]
    bt = gen.block_table(cfg, ctx)
    kb, vb = gen.synthetic_cache(cfg, bt, ctx)
    kf, vf = gen.bits_to_f32(kb), gen.bits_to_f32(vb)
    x = gen.hidden(cfg, nb)
    if ready:
        ready()
    t0 = time.perf_counter()
    oracle.layer_decode(cfg.dims(), w, x, ctx, kf, vf, bt.table, mode=oracle.EXACT)
    dt = time.perf_counter() - t0
    return {"value": round(nb / dt, 3), "unit": "tokens/s", "cores": 1,
            "sample": f"first {nb} sequences of the 7B decode step (contexts "
                      f"{', '.join(str(int(c)) for c in ctx)}), exact mode, {dt:.2f} s"}


def cpu_child(kind: str):
    """Start cpu_sample in a child process pinned to one OpenMP thread; the
    caller starts it before touching the GPU and collects it with
    cpu_child_result (the child never touches the GPU).  The child builds its
    inputs, then waits for a line on its stdin before its timed part, so the
    caller releases it only while its own process is idle."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-sample", kind],
                            stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                            stderr=subprocess.PIPE, text=True, env=env)


def cpu_child_result(proc) -> dict:
    """Release the child's timed part and wait for its JSON line (the caller
    does nothing else meanwhile)."""
    try:
        out, err = proc.communicate(input="go\n", timeout=600)
    except Exception as e:   # noqa: BLE001
        proc.kill()
        return {"error": str(e)}
    if proc.returncode != 0:
        return {"error": (err or "")[-300:]}
    return json.loads(out.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mode", choices=["fused", "unfused"], default="fused")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-int8", action="store_true", help="skip the INT8-cache decode line")
    ap.add_argument("--no-verify", action="store_true", help="skip the q_len 4 verification line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="no clock-sampler child (for runs under a profiler, whose preloaded "
                         "library initialises the GPU before this script starts, after which "
                         "no child program may be started)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="prefix length of the CPU-oracle sample")
    ap.add_argument("--cpu-sample", choices=["tiny", "decode"], default=None,
                    help=argparse.SUPPRESS)   # the one-thread CPU child (no GPU use)
    ap.add_argument("--clock-sampler", action="store_true",
                    help=argparse.SUPPRESS)   # the clock-reading child (no GPU use)
    args = ap.parse_args()
    if args.cpu_sample:
        print(json.dumps(cpu_sample(args.cpu_sample, ready=sys.stdin.readline)), flush=True)
        return
    if args.clock_sampler:
        clock_sampler_child()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer is "
              "built and measured on a single MI355X; across GPUs decode would shard by "
              "sequence (no exchange) or by KV head and FFN columns with one all-reduce after "
              "O and one after down, none of which is built here", file=sys.stderr)
        sys.exit(2)

    # children first: nothing is started from this process once it has
    # touched the GPU
    clocks = NoClock() if args.no_clock else ClockSampler()
    host = host_cpu()
    children = {}
    if not args.no_cpu_baseline:
        children["tiny"] = cpu_child("tiny")
        if not args.no_decode:
            children["decode"] = cpu_child("decode")

    import numpy as np
    import torch

    from transformer_decoder_layer_residual_amd import binding as dl
    from transformer_decoder_layer_residual_amd import inputs as gen
    from transformer_decoder_layer_residual_amd.harness import (DeviceLayer, cache_dev, i32,
                                                                to_dev)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dl.lib()   # fail loudly now if the HIP library is missing
    stream = torch.cuda.current_stream()
    mode = dl.DL_FUSED if args.mode == "fused" else dl.DL_UNFUSED

    # ------------------------------------------------------------------ prefill
    cfg = gen.CONFIGS[2]
    pb = gen.prefill_batch(cfg)
    T = pb.T
    log(f"[bench] generating {cfg.name} inputs")
    t0 = time.time()
    w_host = gen.weights(cfg)
    x_host = gen.hidden(cfg, T)
    bt = gen.block_table(cfg, pb.lens)
    kbits, vbits = gen.empty_cache(cfg, bt.num_blocks)
    # one RoPE table long enough for the prefill and for 4096-token decode contexts
    layer = DeviceLayer.build(cfg, max_pos=max(T, 4096), w_host=w_host)
    x = to_dev(x_host, torch.float32)
    y = torch.empty_like(x)
    kc, vc = cache_dev(kbits), cache_dev(vbits)
    btd = i32(bt.table)
    pos, seq, cu = i32(pb.positions), i32(pb.seq_of_token), i32(pb.cu_seqlens)
    ws_bytes = dl.dl_layer_workspace_size(layer.dims, T, pb.B, pb.max_seqlen, 0, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; workspace {ws_bytes / 2**20:.0f} MiB")

    def step():
        dl.dl_layer_prefill(layer.dims, layer.w, layer.cs, x, y, pos, seq, cu, pb.max_seqlen, kc,
                            vc, btd, mode=mode, ws=ws)

    flush = Flusher()
    warm_up(step, args.warmup, stream)
    ms, p10, p90 = time_cold(step, args.steps, stream, flush)
    tok_s = T / (ms * 1e-3)
    warm_ms = time_launches(step, args.steps, stream)
    H, Hq, D, I = cfg.hidden, cfg.n_q_heads, cfg.head_dim, cfg.intermediate
    Hkv = cfg.n_kv_heads
    gemm_flops = 2.0 * T * H * ((Hq + 2 * Hkv) * D + Hq * D + 2 * I + I)
    attn_flops = 4.0 * Hq * D * float((pb.lens.astype(np.int64) * (pb.lens + 1) // 2).sum())
    layer_flops = gemm_flops + attn_flops
    log(f"[bench] prefill: {ms:.3f} ms/step (median, cold; p10 {p10:.3f}, p90 {p90:.3f}; "
        f"back-to-back {warm_ms:.3f}), {tok_s:,.0f} tokens/s, "
        f"{layer_flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s")

    # dominant kernel: gate/up GEMM with the SiLU*mul epilogue, timed with HIP
    # events around its own launch inside the layer's step-by-step chain (the
    # same kernels as the fused call), so caches hold what they hold in a layer
    kc2, vc2 = cache_dev(kbits), cache_dev(vbits)
    pairs = []
    for i in range(max(args.steps // 2, 10) + 2):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        layer.steps_prefill(x, pb, kc2, vc2, btd, gu_events=ev)
        if i >= 2:
            pairs.append(ev)
    torch.cuda.synchronize()
    gu_ms = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
    del kc2, vc2
    gu_flops = 2.0 * T * (2 * I) * H
    gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
    gu_traffic = load_traffic("gemm_gateup_silu_prefill")
    log(f"[bench] gate/up GEMM: {gu_ms:.3f} ms, {gu_tf:.0f} TFLOP/s "
        f"({100 * gu_tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
    # graphics clock under the prefill step (sampled after the timed region):
    # the published peaks are at 2400 MHz
    clk_prefill = clocks.under(step, stream)
    log(f"[bench] graphics clock under the prefill step: {clk_prefill} MHz")

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": "llama2-7b-layer-prefill", "batch": 1, "seq_len": T,
                   "hidden": H, "heads": f"{Hq}/{Hkv}x{D}", "intermediate": I,
                   "mode": args.mode},
        "cache_state": "cold: 1 GiB written before every step, outside its events; "
                       "ms_per_step is the median over the steps",
        "warm_back_to_back_ms_per_step": round(warm_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm gate/up + SiLU*mul",
                     "cache_state": "inside back-to-back step-by-step layer chains",
                     "achieved": round(gu_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / PEAK_BF16_TFLOPS, 4), "traffic": gu_traffic,
                     "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 4),
                     "frac_at_measured_clock": (round(gu_tf / (PEAK_BF16_TFLOPS * clk_prefill
                                                               / SPEC_CLOCK_MHZ), 4)
                                                if clk_prefill else None)},
        "clock": {"spec_mhz": SPEC_CLOCK_MHZ, "prefill_step_mhz": clk_prefill,
                  "source": "amd-smi metric -c (run by a child process started before the GPU "
                            "is touched), mean over the XCD clock domains, sampled while the step "
                            "repeats after its timed region"},
        "step_ms_percentiles": {"p10": round(p10, 4), "p50": round(ms, 4), "p90": round(p90, 4),
                                "steps": args.steps},
        "layer": {"flops_per_step": layer_flops,
                  "achieved_tflops": round(layer_flops / (ms * 1e-3) / 1e12, 1),
                  "frac_of_bf16_peak": round(layer_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                             4)},
    }
    del ws, kc, vc
    torch.cuda.empty_cache()

    # ------------------------------------------- 8B-GQA ragged prefill batch
    def run_prefill_gqa():
        """Llama-3-8B-shaped GQA layer (32/8 heads x 128, I 14336, theta 5e5):
        one prefill call over 8 packed sequences of U{256..1024} tokens."""
        c4 = gen.CONFIGS[4]
        pb4 = gen.prefill_batch(c4)
        T4 = pb4.T
        log(f"[bench] generating {c4.name} prefill inputs (T={T4}, lens {pb4.lens.tolist()})")
        lay = DeviceLayer.build(c4, max_pos=int(pb4.lens.max()) + 1)
        x4 = to_dev(gen.hidden(c4, T4), torch.float32)
        y4 = torch.empty_like(x4)
        bt4 = gen.block_table(c4, pb4.lens)
        kb, vb = gen.empty_cache(c4, bt4.num_blocks)
        kc4, vc4 = cache_dev(kb), cache_dev(vb)
        bt4d = i32(bt4.table)
        p4, s4, cu4 = i32(pb4.positions), i32(pb4.seq_of_token), i32(pb4.cu_seqlens)
        ws4 = torch.empty(dl.dl_layer_workspace_size(lay.dims, T4, pb4.B, pb4.max_seqlen, 0, mode),
                          dtype=torch.uint8, device="cuda:0")

        def step4():
            dl.dl_layer_prefill(lay.dims, lay.w, lay.cs, x4, y4, p4, s4, cu4, pb4.max_seqlen, kc4,
                                vc4, bt4d, mode=mode, ws=ws4)

        warm_up(step4, args.warmup, stream)
        ms4, q10, q90 = time_cold(step4, args.steps, stream, flush)
        warm4 = time_launches(step4, args.steps, stream)
        kc5, vc5 = cache_dev(kb), cache_dev(vb)
        pairs4 = []
        for i in range(max(args.steps // 2, 10) + 2):
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            lay.steps_prefill(x4, pb4, kc5, vc5, bt4d, gu_events=ev)
            if i >= 2:
                pairs4.append(ev)
        torch.cuda.synchronize()
        gu4_ms = sum(a.elapsed_time(b) for a, b in pairs4) / len(pairs4)
        H4, Hq4, Hkv4, D4, I4 = c4.hidden, c4.n_q_heads, c4.n_kv_heads, c4.head_dim, \
            c4.intermediate
        g_fl = 2.0 * T4 * H4 * ((Hq4 + 2 * Hkv4) * D4 + Hq4 * D4 + 3 * I4)
        a_fl = 4.0 * Hq4 * D4 * float((pb4.lens.astype(np.int64) * (pb4.lens + 1) // 2).sum())
        gu4_fl = 2.0 * T4 * (2 * I4) * H4
        gu4_tf = gu4_fl / (gu4_ms * 1e-3) / 1e12
        out = {"workload": "llama3-8b-gqa-layer-prefill-b8-ragged", "batch": pb4.B,
               "tokens": T4, "lens": pb4.lens.tolist(),
               "value": round(T4 / (ms4 * 1e-3), 1), "unit": "tokens/s",
               "ms_per_step": round(ms4, 4),
               "cache_state": "cold (1 GiB written before every step; median)",
               "step_ms_p10_p90": [round(q10, 4), round(q90, 4)],
               "warm_back_to_back_ms_per_step": round(warm4, 4),
               "layer": {"flops_per_step": g_fl + a_fl,
                         "achieved_tflops": round((g_fl + a_fl) / (ms4 * 1e-3) / 1e12, 1),
                         "frac_of_bf16_peak": round((g_fl + a_fl) / (ms4 * 1e-3) / 1e12
                                                    / PEAK_BF16_TFLOPS, 4)},
               "roofline": {"bound": "mfma", "kernel": "gemm gate/up + SiLU*mul",
                            "cache_state": "inside back-to-back step-by-step layer chains",
                            "achieved": round(gu4_tf, 1), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(gu4_tf / PEAK_BF16_TFLOPS, 4),
                            "traffic": load_traffic("gemm_gateup_silu_prefill_8b"),
                            "flops_per_launch": gu4_fl,
                            "avg_launch_ms": round(gu4_ms, 4)}}
        log(f"[bench] 8B GQA prefill B8 ragged (T={T4}): {ms4:.3f} ms/step (cold median; "
            f"back-to-back {warm4:.3f}), {T4 / (ms4 * 1e-3):,.0f} tokens/s; gate/up "
            f"{gu4_ms:.3f} ms = {gu4_tf:.0f} TFLOP/s")
        del kc4, vc4, kc5, vc5, ws4, lay
        torch.cuda.empty_cache()
        return out

    result["prefill_gqa_8b"] = run_prefill_gqa()

    # ------------------------------------------------------------------ decode
    def run_decode(int8: bool):
        dcfg = gen.CONFIGS[3]          # same layer shape (and weights) as the prefill
        ctx = gen.decode_context_lens(dcfg)
        B = ctx.size
        kind = "INT8" if int8 else "bf16"
        log(f"[bench] generating {dcfg.name} {kind} cache (B={B}, mean ctx {ctx.mean():.0f})")
        dbt = gen.block_table(dcfg, ctx)
        host_cache = gen.synthetic_cache_q8(dcfg, dbt, ctx) if int8 else \
            gen.synthetic_cache(dcfg, dbt, ctx)
        caches = [cache_dev(a) for a in host_cache]
        del host_cache
        kc, vc = caches[0], caches[1]
        sc = {"k_scale": caches[2], "v_scale": caches[3]} if int8 else {}
        dbtd = i32(dbt.table)
        xd = to_dev(gen.hidden(dcfg, B), torch.float32)
        yd = torch.empty_like(xd)
        max_ctx = int(ctx.max())
        dpos, dctx = i32(ctx - 1), i32(ctx)
        dws_n = dl.dl_layer_workspace_size(layer.dims, B, B, 0, max_ctx, mode)
        dws = torch.empty(dws_n, dtype=torch.uint8, device="cuda:0")

        def dstep():
            dl.dl_layer_decode(layer.dims, layer.w, layer.cs, xd, yd, dpos, dctx, max_ctx, kc,
                               vc, dbtd, mode=mode, ws=dws, **sc)

        warm_up(dstep, args.warmup, stream)
        dms, dp10, dp90 = time_cold(dstep, args.steps, stream, flush)
        dwarm = time_launches(dstep, args.steps, stream)
        # the same step replayed as one HIP graph (dl_layer_decode_graph_create)
        side = torch.cuda.Stream()
        graph = dl.DecodeGraph(layer.dims, layer.w, layer.cs, xd, yd, dpos, dctx, max_ctx, kc, vc,
                               dbtd, side, ws=dws,
                               **({"k_scale": sc["k_scale"], "v_scale": sc["v_scale"]} if int8
                                  else {}))
        for _ in range(args.warmup):
            graph.launch()
        side.synchronize()
        gms = time_launches(graph.launch, args.steps, side)
        graph.close()
        # dominant kernel: paged decode attention (split + combine)
        q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda:0").normal_()
        ao = torch.empty_like(q)
        aws_n = dl.lib().dl_attn_decode_workspace_size(B, Hq, Hkv, D, max_ctx, dcfg.block_size)
        aws = torch.empty(aws_n, dtype=torch.uint8, device="cuda:0")

        def dattn():
            dl.dl_attn_decode_paged(q, kc, vc, dbtd, dctx, max_ctx, ao, ws=aws, **sc)

        for _ in range(3):
            dattn()
        a_ms, _, _ = time_cold(dattn, max(args.steps, 20), stream, flush)
        a_warm = time_launches(dattn, max(args.steps, 20), stream)
        # per cached token and kv head: K and V rows of D elements (+ a 4-byte
        # scale each for INT8)
        row_bytes = 2.0 * ((D + 4) if int8 else D * 2)
        kv_bytes = float(ctx.astype(np.int64).sum()) * Hkv * row_bytes
        a_bytes = kv_bytes + 2.0 * B * Hq * D * 2
        a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
        w_bytes = 2.0 * (H * (Hq + 2 * Hkv) * D + Hq * D * H + 3 * H * I)
        step_bytes = w_bytes + kv_bytes
        out = {
            "workload": "llama2-7b-layer-decode" + ("-kv-int8" if int8 else ""), "batch": B,
            "context": "uniform 128..4096 (mean %.0f)" % ctx.mean(),
            "kv_cache": "int8 codes + fp32 per-token scales" if int8 else "bf16",
            "value": round(B / (dms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(dms, 4),
            "cache_state": "cold (1 GiB written before every step; median)",
            "step_ms_p10_p90": [round(dp10, 4), round(dp90, 4)],
            "warm_back_to_back_ms_per_step": round(dwarm, 4),
            "graph_ms_per_step": round(gms, 4),
            "graph_cache_state": "warm (back-to-back replays)",
            "graph_tokens_per_s": round(B / (gms * 1e-3), 1),
            "step_hbm_frac": round(step_bytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "paged decode attention (split-KV + combine)"
                         + (" over INT8 blocks" if int8 else ""),
                         "achieved": round(a_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(a_gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("attn_decode_paged_int8" if int8
                                                 else "attn_decode_paged"),
                         "bytes_per_launch": a_bytes, "avg_launch_ms": round(a_ms, 4),
                         "cache_state": "cold (median of flushed launches)",
                         "warm_back_to_back_ms": round(a_warm, 4)},
        }
        if not int8:
            clk = clocks.under(dstep, stream)
            result["clock"]["decode_step_mhz"] = clk
            log(f"[bench] graphics clock under the decode step: {clk} MHz")
        log(f"[bench] decode ({kind} cache): {dms:.3f} ms/step, {B / (dms * 1e-3):,.0f} "
            f"tokens/s (graph {gms:.3f} ms); attention {a_ms:.3f} ms = {a_gbs:,.0f} GB/s")
        del caches, kc, vc, sc, dws, aws
        torch.cuda.empty_cache()
        return out

    # ------------------------------------------- verification step (q_len > 1)
    def run_verify(qlen: int):
        """Every sequence of the decode workload verifies qlen candidate tokens
        in one layer step (attention over the paged cache with per-sequence
        query lengths)."""
        dcfg = gen.CONFIGS[3]
        ctx = gen.decode_context_lens(dcfg)   # context lengths after the step
        B = ctx.size
        log(f"[bench] generating {dcfg.name} cache for {qlen}-token verification")
        dbt = gen.block_table(dcfg, ctx)
        kb, vb = gen.synthetic_cache(dcfg, dbt, ctx - (qlen - 1))   # positions before the step
        kc, vc = cache_dev(kb), cache_dev(vb)
        del kb, vb
        qb = gen.packed(np.full(B, qlen, np.int32))
        T = qb.T
        xq = to_dev(gen.hidden(dcfg, T, step=3), torch.float32)
        dbtd = i32(dbt.table)
        vws_n = dl.lib().dl_layer_decode_qlens_workspace_size(layer.dims, T, B, qlen,
                                                              int(ctx.max()))
        vws = torch.empty(vws_n, dtype=torch.uint8, device="cuda:0")

        # per-token positions, sequence ids, cu_q and context lengths resident
        # on the device before the timed region, like every other input
        vpos = i32((np.repeat(ctx - qb.lens, qb.lens) + qb.positions).astype(np.int32))
        vseq, vcu, vctx = i32(qb.seq_of_token), i32(qb.cu_seqlens), i32(ctx)
        yq = torch.empty_like(xq)

        def vstep():
            dl.dl_layer_decode_qlens(layer.dims, layer.w, layer.cs, xq, yq, vpos, vseq, vcu, vctx,
                                     qb.max_seqlen, int(ctx.max()), kc, vc, dbtd, ws=vws)

        warm_up(vstep, args.warmup, stream)
        vms, _, _ = time_cold(vstep, args.steps, stream, flush)
        q = torch.empty(T, Hq, D, dtype=torch.bfloat16, device="cuda:0").normal_()
        ao = torch.empty_like(q)
        cu, dctx = i32(qb.cu_seqlens), i32(ctx)
        aws_n = dl.lib().dl_attn_paged_qlens_workspace_size(B, T, Hq, Hkv, D, qlen, int(ctx.max()),
                                                            dcfg.block_size)
        aws = torch.empty(aws_n, dtype=torch.uint8, device="cuda:0")

        def vattn():
            dl.dl_attn_paged_qlens(q, kc, vc, dbtd, cu, dctx, qlen, int(ctx.max()), ao, ws=aws)

        for _ in range(3):
            vattn()
        a_ms, _, _ = time_cold(vattn, max(args.steps, 20), stream, flush)
        kv_bytes = 2.0 * float(ctx.astype(np.int64).sum()) * Hkv * D * 2
        a_bytes = kv_bytes + 2.0 * T * Hq * D * 2
        a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
        out = {
            "workload": "llama2-7b-layer-verify-%d" % qlen, "batch": B, "q_len": qlen,
            "context": "uniform 128..4096 (mean %.0f) after the step" % ctx.mean(),
            "value": round(T / (vms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(vms, 4),
            "cache_state": "cold (1 GiB written before every step; median)",
            "roofline": {"bound": "hbm", "kernel": "paged attention, q_len %d (split-KV + combine)"
                         % qlen, "cache_state": "cold (median of flushed launches)",
                         "achieved": round(a_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(a_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "bytes_per_launch": a_bytes, "avg_launch_ms": round(a_ms, 4)},
        }
        log(f"[bench] verify q_len {qlen}: {vms:.3f} ms/step, {T / (vms * 1e-3):,.0f} tokens/s; "
            f"attention {a_ms:.3f} ms = {a_gbs:,.0f} GB/s")
        del kc, vc, vws, aws
        torch.cuda.empty_cache()
        return out

    # --------------------------------- small-batch GQA decode, eager vs graph
    def run_small_decode():
        """Llama-3-8B-shaped layer (random weights), B8 at the contexts its own
        workload reaches after prefill (U{256..1024} + 64): a step of ~80 us
        where host launch gaps show."""
        c4 = gen.CONFIGS[4]
        lay = DeviceLayer.build(c4, max_pos=1200)
        ctx = (gen.prefill_batch(c4).lens + 64).astype(np.int32)
        B4 = ctx.size
        bt4 = gen.block_table(c4, ctx)
        kb, vb = gen.synthetic_cache(c4, bt4, ctx)
        kc4, vc4 = cache_dev(kb), cache_dev(vb)
        del kb, vb
        bt4d = i32(bt4.table)
        x4 = to_dev(gen.hidden(c4, B4, step=9), torch.float32)
        y4 = torch.empty_like(x4)
        p4, c4d = i32(ctx - 1), i32(ctx)
        mx = int(ctx.max())
        ws4 = torch.empty(dl.dl_layer_workspace_size(lay.dims, B4, B4, 0, mx, mode),
                          dtype=torch.uint8, device="cuda:0")

        def step4():
            dl.dl_layer_decode(lay.dims, lay.w, lay.cs, x4, y4, p4, c4d, mx, kc4, vc4, bt4d,
                               ws=ws4)

        for _ in range(args.warmup):
            step4()
        torch.cuda.synchronize()
        ems = time_launches(step4, max(args.steps, 50), stream)
        side = torch.cuda.Stream()
        g4 = dl.DecodeGraph(lay.dims, lay.w, lay.cs, x4, y4, p4, c4d, mx, kc4, vc4, bt4d, side,
                            ws=ws4)
        for _ in range(args.warmup):
            g4.launch()
        side.synchronize()
        gms = time_launches(g4.launch, max(args.steps, 50), side)
        ems_sync = time_synced(step4, max(args.steps, 50), stream)
        gms_sync = time_synced(g4.launch, max(args.steps, 50), side)
        g4.close()
        H4, Hq4, Hkv4, D4, I4 = c4.hidden, c4.n_q_heads, c4.n_kv_heads, c4.head_dim, \
            c4.intermediate
        w_bytes = 2.0 * (H4 * (Hq4 + 2 * Hkv4) * D4 + Hq4 * D4 * H4 + 3 * H4 * I4)
        kv_bytes = 2.0 * float(ctx.astype(np.int64).sum()) * Hkv4 * D4 * 2
        ecold, _, _ = time_cold(step4, max(args.steps, 50), stream, flush)
        out = {"workload": "llama3-8b-layer-decode-b8", "batch": B4,
               "cache_state": "warm (back-to-back) unless named cold",
               "cold_eager_ms_per_step": round(ecold, 4),
               "context": "prefill lengths U{256..1024} + 64 (mean %.0f)" % ctx.mean(),
               "eager_ms_per_step": round(ems, 4), "graph_ms_per_step": round(gms, 4),
               "synced_eager_ms_per_step": round(ems_sync, 4),
               "synced_graph_ms_per_step": round(gms_sync, 4),
               "eager_tokens_per_s": round(B4 / (ems * 1e-3), 1),
               "graph_tokens_per_s": round(B4 / (gms * 1e-3), 1),
               "graph_step_hbm_frac": round((w_bytes + kv_bytes) / (gms * 1e-3) / 1e9
                                            / PEAK_HBM_GBS, 4)}
        log(f"[bench] 8B decode B{B4}: eager {ems:.4f} ms, graph {gms:.4f} ms per step; with a "
            f"host sync per step: eager {ems_sync:.4f} ms, graph {gms_sync:.4f} ms")
        del kc4, vc4, ws4

        # The workload as a sequence: 128 decode steps on the cache its prefill
        # left, contexts S_b+1 .. S_b+128 (each step writes its token's K/V into
        # the paged cache before attending); HIP events around every step,
        # median over the 128 steps.
        lens = gen.prefill_batch(c4).lens.astype(np.int32)
        btS = gen.block_table(c4, lens + 128)
        kb, vb = gen.synthetic_cache(c4, btS, lens + 1)       # positions < S_b
        kcS, vcS = cache_dev(kb), cache_dev(vb)
        del kb, vb
        btSd = i32(btS.table)
        mxS = int(lens.max()) + 128
        wsS = torch.empty(dl.dl_layer_workspace_size(lay.dims, B4, B4, 0, mxS, mode),
                          dtype=torch.uint8, device="cuda:0")
        posS = [i32(lens + i) for i in range(128)]
        ctxS = [i32(lens + i + 1) for i in range(128)]

        def run_seq(evs=None):
            for i in range(128):
                if evs:
                    evs[i][0].record(stream)
                dl.dl_layer_decode(lay.dims, lay.w, lay.cs, x4, y4, posS[i], ctxS[i], mxS, kcS,
                                   vcS, btSd, ws=wsS)
                if evs:
                    evs[i][1].record(stream)

        run_seq()                      # warm-up pass: writes the K/V the timed pass rewrites
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(128)]
        run_seq(evs)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        med, p10, p90 = ts[64], ts[12], ts[115]
        out["steps128"] = {"context": "S_b+1 .. S_b+128, S_b ~ U{256..1024}",
                           "median_ms_per_step": round(med, 4), "p10_ms": round(p10, 4),
                           "p90_ms": round(p90, 4),
                           "median_tokens_per_s": round(B4 / (med * 1e-3), 1)}
        log(f"[bench] 8B decode B{B4}, 128 steps from the prefill lengths: median {med:.4f} ms "
            f"(p10 {p10:.4f}, p90 {p90:.4f})")
        del kcS, vcS, wsS, lay
        torch.cuda.empty_cache()
        return out

    # ------------------------------------------------ 70B-shaped GQA decode
    def run_gqa_decode():
        """Llama-2-70B-shaped layer (random weights, 64/8 heads): decode at B4
        with 4096-token contexts and at B1 with 32768.  At these batches the
        step reads every weight once; attention reads the whole KV cache."""
        c5 = gen.CONFIGS[5]
        lay = DeviceLayer.build(c5, max_pos=max(c for _, c in c5.extra["cases"]) + 1)
        H5, Hq5, Hkv5, D5, I5 = c5.hidden, c5.n_q_heads, c5.n_kv_heads, c5.head_dim, \
            c5.intermediate
        w_bytes = 2.0 * (H5 * (Hq5 + 2 * Hkv5) * D5 + Hq5 * D5 * H5 + 3 * H5 * I5)
        outs = []
        for case in range(len(c5.extra["cases"])):
            ctx = gen.decode_context_lens(c5, case)
            B5, mx = ctx.size, int(ctx.max())
            bt5 = gen.block_table(c5, ctx)
            kb, vb = gen.synthetic_cache(c5, bt5, ctx, case=case)
            kc5, vc5 = cache_dev(kb), cache_dev(vb)
            del kb, vb
            bt5d = i32(bt5.table)
            x5 = to_dev(gen.hidden(c5, B5, step=11 + case), torch.float32)
            y5 = torch.empty_like(x5)
            p5, c5d = i32(ctx - 1), i32(ctx)
            ws5 = torch.empty(dl.dl_layer_workspace_size(lay.dims, B5, B5, 0, mx, mode),
                              dtype=torch.uint8, device="cuda:0")

            def step5():
                dl.dl_layer_decode(lay.dims, lay.w, lay.cs, x5, y5, p5, c5d, mx, kc5, vc5, bt5d,
                                   ws=ws5)

            warm_up(step5, args.warmup, stream)
            ems, _, _ = time_cold(step5, max(args.steps, 20), stream, flush)
            ewarm = time_launches(step5, max(args.steps, 20), stream)
            side = torch.cuda.Stream()
            g5 = dl.DecodeGraph(lay.dims, lay.w, lay.cs, x5, y5, p5, c5d, mx, kc5, vc5, bt5d,
                                side, ws=ws5)
            for _ in range(args.warmup):
                g5.launch()
            side.synchronize()
            gms = time_launches(g5.launch, max(args.steps, 20), side)
            g5.close()
            q5 = torch.empty(B5, Hq5, D5, dtype=torch.bfloat16, device="cuda:0").normal_()
            ao = torch.empty_like(q5)
            aws = torch.empty(dl.lib().dl_attn_decode_workspace_size(B5, Hq5, Hkv5, D5, mx,
                                                                     c5.block_size),
                              dtype=torch.uint8, device="cuda:0")

            def attn5():
                dl.dl_attn_decode_paged(q5, kc5, vc5, bt5d, c5d, mx, ao, ws=aws)

            for _ in range(3):
                attn5()
            a_ms, _, _ = time_cold(attn5, max(args.steps, 20), stream, flush)
            a_warm = time_launches(attn5, max(args.steps, 20), stream)
            kv_bytes = 2.0 * float(ctx.astype(np.int64).sum()) * Hkv5 * D5 * 2
            a_bytes = kv_bytes + 2.0 * B5 * Hq5 * D5 * 2
            a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
            # the FFN's two projections alone (the same kernels the step runs at
            # this batch); each streams more weight bytes than the MALL holds
            n2 = torch.empty(B5, H5, dtype=torch.bfloat16, device="cuda:0").normal_()
            act = torch.empty(B5, I5, dtype=torch.bfloat16, device="cuda:0")
            res5 = torch.empty(B5, H5, dtype=torch.float32, device="cuda:0").normal_()
            fo5 = torch.empty_like(res5)

            def gu5():
                dl.dl_gate_up_silu(n2, lay.w["wg"], lay.w["wu"], act)

            def dn5():
                dl.dl_down_residual(act, lay.w["wd"], fo5, residual=res5)

            for _ in range(3):
                gu5()
                dn5()
            gu_ms, _, _ = time_cold(gu5, max(args.steps, 20), stream, flush)
            dn_ms, _, _ = time_cold(dn5, max(args.steps, 20), stream, flush)
            gu_bytes = 2.0 * I5 * H5 * 2 + B5 * H5 * 2 + B5 * I5 * 2
            dn_bytes = 1.0 * H5 * I5 * 2 + B5 * I5 * 2 + 2.0 * B5 * H5 * 4
            f_gbs = (gu_bytes + dn_bytes) / ((gu_ms + dn_ms) * 1e-3) / 1e9
            ffn = {"kernel": "gate/up + SiLU*mul and down + residual (row-block weight stream)",
                   "cache_state": "cold (median of flushed launches)",
                   "achieved": round(f_gbs, 1), "unit": "GB/s",
                   "frac": round(f_gbs / PEAK_HBM_GBS, 4),
                   "gate_up": {"avg_launch_ms": round(gu_ms, 4), "bytes_per_launch": gu_bytes,
                               "traffic": load_traffic("gemm_gateup_silu_decode_70b"),
                               "frac": round(gu_bytes / (gu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                   "down": {"avg_launch_ms": round(dn_ms, 4), "bytes_per_launch": dn_bytes,
                            "frac": round(dn_bytes / (dn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
            outs.append({
                "workload": "llama2-70b-layer-decode-b%d-ctx%d" % (B5, mx), "batch": B5,
                "context": mx, "value": round(B5 / (ems * 1e-3), 1), "unit": "tokens/s",
                "ms_per_step": round(ems, 4),
                "cache_state": "cold (1 GiB written before every step; median)",
                "warm_back_to_back_ms_per_step": round(ewarm, 4),
                "graph_ms_per_step": round(gms, 4),
                "graph_step_hbm_frac": round((w_bytes + kv_bytes) / (gms * 1e-3) / 1e9
                                             / PEAK_HBM_GBS, 4),
                "attention": {"kernel": "paged decode attention, 8-head query groups "
                              "(split-KV + combine)",
                              "cache_state": "cold (median of flushed launches)",
                              "warm_back_to_back_ms": round(a_warm, 4),
                              "warm_back_to_back_gbs": round(a_bytes / (a_warm * 1e-3) / 1e9, 1),
                              "achieved": round(a_gbs, 1),
                              "unit": "GB/s", "frac": round(a_gbs / PEAK_HBM_GBS, 4),
                              "bytes_per_launch": a_bytes, "avg_launch_ms": round(a_ms, 4)},
                "ffn": ffn})
            log(f"[bench] 70B decode B{B5} x {mx}: eager {ems:.4f} ms, graph {gms:.4f} ms per "
                f"step ({outs[-1]['graph_step_hbm_frac'] * 100:.0f}% of HBM peak); attention "
                f"{a_ms * 1e3:.1f} us = {a_gbs:,.0f} GB/s; FFN gate/up {gu_ms * 1e3:.1f} us + "
                f"down {dn_ms * 1e3:.1f} us = {f_gbs:,.0f} GB/s")
            del kc5, vc5, ws5, aws, n2, act, res5, fo5
            torch.cuda.empty_cache()
        del lay
        torch.cuda.empty_cache()
        return outs

    if not args.no_decode:
        result["decode_gqa_70b"] = run_gqa_decode()
        result["decode_small_batch"] = run_small_decode()
        result["decode"] = run_decode(False)
        if not args.no_int8:
            result["decode_kv_int8"] = run_decode(True)
        if not args.no_verify:
            result["verify_qlen4"] = run_verify(4)

    # ------------------------------------------------------------ cpu baseline
    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_tokens, T)
        sub = gen.packed([n])
        log(f"[bench] CPU oracle on the first {n} tokens")
        t0 = time.time()
        oracle.layer_prefill(cfg.dims(), w_host, x_host[:n], sub.positions, sub.seq_of_token,
                             sub.cu_seqlens, mode=oracle.EXACT)
        dt = time.time() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        result["cpu_baseline"] = {
            "value": round(n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of the {T} prefill tokens, same weights, exact fp32/fp64 "
                      f"mode, {dt:.1f} s", "host": host}
        # the tiny fp32 layer (prefill of 32 tokens + 8 decode steps) on all
        # threads here and on one thread in a child process; the 7B decode
        # step for 4 sequences on one thread
        tiny = cpu_sample("tiny")
        tiny1 = cpu_child_result(children["tiny"])
        result["cpu_baseline_tiny"] = {
            "unit": "tokens/s", "kind": "oracle",
            "sample": "tiny fp32 layer: prefill of 32 tokens, then 8 decode steps; 5 timed "
                      "passes after an untimed one",
            "all_threads": {"cores": cores, **tiny}, "one_thread": {"cores": 1, **tiny1}}
        # the decode step too: the oracle's layer step for the first sequences
        # of the 7B decode workload, over their own cache blocks (the bf16
        # cache's values in fp32), same weights
        if not args.no_decode:
            dcfg = gen.CONFIGS[3]
            nb = 16
            dctx = gen.decode_context_lens(dcfg)[:nb]
            dbt = gen.block_table(dcfg, dctx)
            kb, vb = gen.synthetic_cache(dcfg, dbt, dctx)
            kf, vf = gen.bits_to_f32(kb), gen.bits_to_f32(vb)
            del kb, vb
            xdh = gen.hidden(dcfg, nb)
            log(f"[bench] CPU oracle decode step for {nb} sequences")
            t0 = time.time()
            oracle.layer_decode(dcfg.dims(), w_host, xdh, dctx, kf, vf, dbt.table,
                                mode=oracle.EXACT)
            ddt = time.time() - t0
            result["cpu_baseline_decode"] = {
                "value": round(nb / ddt, 2), "unit": "tokens/s", "cores": cores,
                "kind": "oracle",
                "sample": f"first {nb} of the 64 sequences of the 7B decode step (contexts "
                          f"{', '.join(str(int(c)) for c in dctx)}), same weights, exact "
                          f"fp32/fp64 mode, {ddt:.2f} s",
                "one_thread": cpu_child_result(children["decode"])}
            del kf, vf
    clocks.close()
    for proc in children.values():
        if proc.poll() is None:
            proc.kill()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
