"""Measurement helpers around rocprofv3 output (kernel-trace stats and PMC
counters) and a layer-bytes driver.

HBM bytes come from the TCC counters FETCH_SIZE and WRITE_SIZE (KiB per
dispatch).  On the MI355X they are calibrated with a plain copy kernel of
known size: a 2 GiB copy reads FETCH_SIZE = 1,048,587 KiB (half of the 2 GiB
read) and WRITE_SIZE = 2,097,152 KiB (exact), so FETCH_SIZE is scaled by 2
and WRITE_SIZE by 1.

Commands (run from the repository root; outputs go where --out says):
  python -m transformer_decoder_layer_residual_amd.profiling stats \
      --csv DIR/x_kernel_stats.csv --out profiles/NAME.md --cmd "COMMAND"
  python -m transformer_decoder_layer_residual_amd.profiling traffic \
      --fetch DIR_F --write DIR_W --out profiles/traffic.json
  python -m transformer_decoder_layer_residual_amd.profiling layer-bytes \
      --mode fused|unfused --calls 3            (run under rocprofv3 --pmc)
  python -m transformer_decoder_layer_residual_amd.profiling bytes-summary \
      --fused-fetch D --fused-write D --unfused-fetch D --unfused-write D \
      --calls 3 --out profiles/NAME.md
  python -m transformer_decoder_layer_residual_amd.profiling ceilings \
      --out profiles/NAME.md                  (achievable rates of the box)
  python -m transformer_decoder_layer_residual_amd.profiling gemm8192 --calls 3
                                              (run under rocprofv3 --pmc)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

FETCH_SCALE = 2.0
WRITE_SCALE = 1.0

# dominant kernels reported by bench.py: key -> (kernel-name regex, sources)
# (rocprofv3 reports some kernel names mangled and some demangled, with
# __bf16 printed as "bool _Accum"; each pattern accepts both forms of the one
# instance the benchmark's roofline line times)
KERNELS = {
    # the 7B prefill gate/up (2048 x 22016 x 4096: 8 x 86 tiles of 512 threads)
    "gemm_gateup_silu_prefill": (r"gemm_pp_kernelILi256ELi64ENS_9MapSwiglu"
                                 r"|gemm_pp_kernel<256, 64, dl::MapSwiglu",
                                 ("gemm_prefill.hpp", "gemm_epi.hpp", "dl_common.hpp"), 688 * 512),
    # the same kernel at the 8B-GQA ragged prefill (6235 x 28672 x 4096: 25 x 112 tiles)
    "gemm_gateup_silu_prefill_8b": (r"gemm_pp_kernelILi256ELi64ENS_9MapSwiglu"
                                    r"|gemm_pp_kernel<256, 64, dl::MapSwiglu",
                                    ("gemm_prefill.hpp", "gemm_epi.hpp", "dl_common.hpp"),
                                    2800 * 512),
    # the 70B-shaped decode gate/up (K = 8192: 16-deep, 8 waves, one row block
    # per workgroup; B4 and B1 calls)
    "gemm_gateup_silu_decode_70b": (r"gemm_row16_kernelILi16ELi8ELi1ENS_9MapSwiglu"
                                    r"|gemm_row16_kernel<16, 8, 1, dl::MapSwiglu",
                                    ("gemm_decode.hpp", "gemm_epi.hpp", "dl_common.hpp")),
    "attn_decode_paged": (r"attn_decode_kernelIDF16bDF16bLi128ELi1E"
                          r"|attn_decode_kernel<bool _Accum, bool _Accum, 128, 1,",
                          ("attn_decode.hip", "dl_common.hpp")),
    "attn_decode_paged_int8": (r"attn_decode_kernelIDF16baLi128ELi1E"
                               r"|attn_decode_kernel<bool _Accum, (signed char, )?128, 1,",
                               ("attn_decode.hip", "dl_common.hpp")),
}


def source_sha(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(PKG, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        out.extend(csv.DictReader(open(f)))
    return out


def _per_kernel(d: str, counter: str):
    """(kernel name, grid size in threads) -> list of per-dispatch counter
    values (KiB)."""
    res = {}
    for r in _rows(d):
        if r["Counter_Name"] != counter:
            continue
        res.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
    return res


def traffic(fetch_dir: str, write_dir: str) -> dict:
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    out = {"fetch_scale": FETCH_SCALE, "write_scale": WRITE_SCALE}
    for key, spec in KERNELS.items():
        rx, srcs = spec[0], spec[1]
        grid = spec[2] if len(spec) > 2 else None   # launch grid of the one workload meant
        names = [n for n in f if re.search(rx, n[0]) and (grid is None or n[1] == grid)]
        if not names:
            continue
        fv = [v for n in names for v in f[n]]
        wv = [v for n in names for v in w.get(n, [])]
        fetch = sum(fv) / len(fv) * 1024 * FETCH_SCALE
        write = (sum(wv) / len(wv) * 1024 * WRITE_SCALE) if wv else 0.0
        out[key] = {"kernel": names[0][0][:160], "grid_threads": names[0][1],
                    "dispatches": len(fv),
                    "fetch_bytes": round(fetch), "write_bytes": round(write),
                    "bytes_per_launch": round(fetch + write),
                    "source_sha": source_sha(*srcs)}
    return out


def layer_bytes(fetch_dir: str, write_dir: str, calls: int) -> dict:
    """HBM bytes of the dl kernels of one layer call (the driver's setup
    kernels and the RoPE table fill are excluded)."""
    def total(d, counter, scale):
        s = 0.0
        per = {}
        for r in _rows(d):
            if r["Counter_Name"] != counter:
                continue
            n = r["Kernel_Name"]
            if "dl" not in n or "rope_table" in n:
                continue
            v = float(r["Counter_Value"]) * 1024 * scale
            s += v
            short = re.sub(r"^_ZN2dl\d+", "", n)[:60]
            per[short] = per.get(short, 0.0) + v
        return s / calls, {k: v / calls for k, v in per.items()}
    fb, fper = total(fetch_dir, "FETCH_SIZE", FETCH_SCALE)
    wb, wper = total(write_dir, "WRITE_SIZE", WRITE_SCALE)
    return {"fetch": fb, "write": wb, "total": fb + wb, "fetch_per_kernel": fper,
            "write_per_kernel": wper}


def counters_md(dirs, out: str, cmd: str, title: str):
    """Per-kernel mean of every counter found under the given rocprofv3 --pmc
    output directories (one directory per pass), as a markdown table; the
    MfmaUtil column is rocprofv3's derived metric (SQ_VALU_MFMA_BUSY_CYCLES
    over GRBM_GUI_ACTIVE x SIMDs, in %)."""
    per = {}
    for d in dirs:
        for r in _rows(d):
            n = re.sub(r"^_ZN2dl\d+", "", r["Kernel_Name"])[:72]
            per.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in per.values() for c in v})
    lines = [f"# {title}", "", "Commands (repository root on the MI355X box; one counter set per run):",
             "", "```", "cd /tmp && export TMPDIR=/tmp && export PYTHONPATH=$REPO", cmd, "```", "",
             "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---:|" + "---:|" * len(names)]
    for n, c in sorted(per.items(), key=lambda kv: -max(len(v) for v in kv[1].values())):
        disp = max(len(v) for v in c.values())
        vals = [f"{sum(c[k]) / len(c[k]):.4g}" if k in c else "" for k in names]
        lines.append(f"| `{n}` | {disp} | " + " | ".join(vals) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic_md(t: dict, out: str):
    lines = ["# HBM traffic of the benchmark's dominant kernels (rocprofv3 PMC)", "",
             "Per-launch bytes = mean over dispatches of FETCH_SIZE x 2 + WRITE_SIZE x 1 (KiB x "
             "1024; scales from a plain 2 GiB copy kernel, which reads FETCH_SIZE = 1,048,587 KiB "
             "and WRITE_SIZE = 2,097,152 KiB).  `source_sha` hashes the kernel's source files; "
             "bench.py reports the figure only while it matches the current source.", "",
             "Commands (repository root on the MI355X box):", "", "```",
             "cd /tmp && export TMPDIR=/tmp",
             "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_f -o bench -- python -u "
             "bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-clock",
             "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_w -o bench -- python -u "
             "bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-clock",
             "python -m transformer_decoder_layer_residual_amd.profiling traffic --fetch "
             "gpurun_out/pmc_f --write gpurun_out/pmc_w --out profiles/traffic.json", "```", "",
             "| key | kernel | dispatches | fetch MB | write MB | bytes/launch MB | source_sha |",
             "|---|---|---:|---:|---:|---:|---|"]
    for k, r in t.items():
        if not isinstance(r, dict):
            continue
        lines.append(f"| {k} | `{r['kernel'][:70]}` | {r['dispatches']} | "
                     f"{r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} | "
                     f"{r['bytes_per_launch'] / 1e6:.1f} | {r['source_sha']} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def stats_md(csv_path: str, out: str, cmd: str, title: str):
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# {title}", "", "Command (repository root on the MI355X box):", "", "```",
             "cd /tmp && export TMPDIR=/tmp", cmd, "```", "",
             "| kernel | calls | avg us | % of GPU time |", "|---|---:|---:|---:|"]
    for r in rows:
        n = re.sub(r"^_ZN2dl\d+", "", r["Name"])[:110]
        lines.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def run_layer(mode: str, calls: int, config: int = 2):
    """One prefill layer call of workload `config` (2: the 7B-shaped B1 x 2048;
    4: the 8B-GQA-shaped 8 ragged sequences), `calls` times, for counters."""
    import torch

    from . import binding as dl
    from . import inputs as gen
    from .harness import DeviceLayer, cache_dev, i32, to_dev
    cfg = gen.CONFIGS[config]
    pb = gen.prefill_batch(cfg)
    layer = DeviceLayer.build(cfg, max_pos=int(pb.lens.max()), w_host=gen.weights(cfg))
    x = to_dev(gen.hidden(cfg, pb.T), torch.float32)
    bt = gen.block_table(cfg, pb.lens)
    kb, vb = gen.empty_cache(cfg, bt.num_blocks)
    kc, vc, btd = cache_dev(kb), cache_dev(vb), i32(bt.table)
    m = dl.DL_FUSED if mode == "fused" else dl.DL_UNFUSED
    n = dl.dl_layer_workspace_size(layer.dims, pb.T, pb.B, pb.max_seqlen, 0, m)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    pos, seq, cu = i32(pb.positions), i32(pb.seq_of_token), i32(pb.cu_seqlens)
    torch.cuda.synchronize()
    for _ in range(calls):
        dl.dl_layer_prefill(layer.dims, layer.w, layer.cs, x, y, pos, seq, cu, pb.max_seqlen, kc,
                            vc, btd, mode=m, ws=ws)
    torch.cuda.synchronize()
    print(f"ran {calls} {mode} prefill layers", file=sys.stderr)


def _probe_lib():
    import ctypes
    path = os.path.join(PKG, "libdl_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "transformer_decoder_layer_residual_amd.build.build()")
    L = ctypes.CDLL(path)
    L.dlp_sink_bytes.restype = ctypes.c_size_t
    L.dlp_mfma_flops.restype = ctypes.c_double
    L.dlp_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    for n, args in (("dlp_stream_read", [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
                    ("dlp_copy", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
                    ("dlp_mfma_loop", [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p])):
        getattr(L, n).restype = ctypes.c_int
        getattr(L, n).argtypes = args
    return L


def _time_ms(fn, n=10, warm=3):
    """Mean milliseconds of n back-to-back calls of fn, HIP events on the
    current stream, after warm untimed calls."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def ceilings(out: str, cmd: str):
    """Achievable rates of this MI355X: a streaming read and a copy of
    buffers far larger than the 256 MB MALL, register-only MFMA loops, and a
    bf16 8192^3 product through this library and through torch (hipBLASLt)."""
    import torch

    from . import binding as dl
    L = _probe_lib()
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.empty(L.dlp_sink_bytes(), dtype=torch.uint8, device="cuda:0")
    rows = []
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)

    def chk(r):
        if r != 0:
            raise RuntimeError(f"probe call failed ({r})")
    best = None
    for bpc in (1, 2, 4, 8, 16):
        for unr in (4, 8, 16):
            ms = _time_ms(lambda: chk(L.dlp_stream_read(buf.data_ptr(), n, sink.data_ptr(), bpc,
                                                        unr, st)), n=5, warm=1)
            if best is None or ms < best[0]:
                best = (ms, bpc, unr)
    ms, bpc, unr = best
    rows.append((f"streaming read, 4 GiB, 16-byte loads (best of 1-16 workgroups per CU x 4-16 "
                 f"loads in flight per lane: {bpc} x {unr})", f"{n / ms / 1e6:,.0f} GB/s",
                 f"{n / ms / 1e6 / 8000:.2f}", "of 8 TB/s"))
    half = n // 2
    src, dst = buf[:half], buf[half:]
    ms = _time_ms(lambda: chk(L.dlp_copy(src.data_ptr(), dst.data_ptr(), half, st)))
    rows.append(("copy, 2 GiB read + 2 GiB written", f"{2 * half / ms / 1e6:,.0f} GB/s",
                 f"{2 * half / ms / 1e6 / 8000:.2f}", "of 8 TB/s"))
    del buf, src, dst
    for kind, name, waves in ((0, "v_mfma_f32_32x32x16_bf16", (1, 2, 3)),
                              (1, "v_mfma_f32_16x16x32_bf16", (1, 2, 4))):
        iters, best = 2000, None
        for wv in waves:
            ms = _time_ms(lambda: chk(L.dlp_mfma_loop(kind, iters, wv, sink.data_ptr(), st)), n=5,
                          warm=1)
            fl = L.dlp_mfma_flops(kind, iters, wv)
            if best is None or fl / ms > best[0]:
                best = (fl / ms, wv)
        rate, wv = best
        rows.append((f"{name}, registers only, 8 chains per wave (best of {list(waves)} waves per "
                     f"SIMD: {wv})", f"{rate / 1e9:,.0f} TFLOP/s", f"{rate / 1e9 / 2500:.2f}",
                     "of 2.5 PFLOP/s"))
    N = 8192
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)
    x = torch.randn(N, N, device="cuda:0", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, N, device="cuda:0", generator=g) * 0.02).to(torch.bfloat16)
    y = torch.empty(N, N, dtype=torch.bfloat16, device="cuda:0")
    fl = 2.0 * N ** 3
    ms = _time_ms(lambda: dl.dl_linear(x, w, y))
    rows.append(("bf16 8192^3 product, this library (dl_linear)", f"{fl / ms / 1e9:,.0f} TFLOP/s",
                 f"{fl / ms / 1e9 / 2500:.2f}", "of 2.5 PFLOP/s"))
    ms = _time_ms(lambda: torch.mm(x, w.t(), out=y))
    rows.append(("bf16 8192^3 product, torch.mm (hipBLASLt)", f"{fl / ms / 1e9:,.0f} TFLOP/s",
                 f"{fl / ms / 1e9 / 2500:.2f}", "of 2.5 PFLOP/s"))
    lines = ["# Achievable rates of the MI355X (measurement kernels and an 8192^3 product)", "",
             "Streaming read and copy: grid-stride kernels of 16-byte accesses over buffers 16x "
             "the 256 MB MALL (the read at 1-16 workgroups of 256 threads per CU and 4-16 "
             "independent loads per lane per trip, the best shown; the copy at 8 workgroups per "
             "CU), mean of back-to-back launches.  MFMA: each wave issues 8 independent "
             "accumulator chains on register operands, one workgroup per CU with 1-4 waves per "
             "SIMD, the best shown.  Products: y = x w^T, x and w 8192 x "
             "8192 bf16 (x ~ N(0,1), w ~ N(0,0.02^2)), mean of 10 launches.  The layer's "
             "fractions of peak are read against these rates.", "",
             "Command (repository root on the MI355X box):", "", "```", cmd, "```", "",
             "| what | rate | fraction | of |", "|---|---:|---:|---|"]
    for r in rows:
        lines.append("| " + " | ".join(r) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[-len(rows) - 2:]))


def projections(out: str, cmd: str):
    """The four prefill projections of the 7B layer (2048 tokens) and of the
    8B-GQA ragged batch (6235 tokens) through this library's entry points
    (with their fused epilogues) and as plain torch.mm products of the same
    shapes (hipBLASLt, no epilogue): cold (1 GiB written and read before
    every launch, median of 15) and back to back (mean of 20)."""
    import torch

    from . import binding as dl
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(*shape, sc=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * sc).to(torch.bfloat16)

    flush_w = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    flush_r = torch.zeros(1 << 28, dtype=torch.int32, device=dev)

    def cold_ms(fn, n=15):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            flush_w.fill_(i)
            flush_r.sum()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return ts[len(ts) // 2]

    shapes = [("llama2-7b, 2048 tokens", 2048, 4096, 32, 32, 128, 11008),
              ("llama3-8b-gqa, 6235 tokens", 6235, 4096, 32, 8, 128, 14336)]
    rows = []
    for label, T, H, Hq, Hkv, D, I in shapes:
        x = rnd(T, H)
        wq, wk, wv = rnd(Hq * D, H, sc=0.02), rnd(Hkv * D, H, sc=0.02), rnd(Hkv * D, H, sc=0.02)
        wqkv = torch.cat([wq, wk, wv], 0)
        wo, wg, wu, wd = (rnd(H, Hq * D, sc=0.02), rnd(I, H, sc=0.02), rnd(I, H, sc=0.02),
                          rnd(H, I, sc=0.02))
        wgu = torch.cat([wg, wu], 0)
        attn, a = rnd(T, Hq * D), rnd(T, I)
        q = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=dev)
        k = torch.empty(T, Hkv, D, dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        cs = torch.empty(4096, D, device=dev)
        dl.dl_rope_table_fill(cs, 4096, D, 1e4)
        pos = (torch.arange(T, device=dev) % 1024).to(torch.int32)
        o = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        act = torch.empty(T, I, dtype=torch.bfloat16, device=dev)
        res = torch.randn(T, H, device=dev, generator=g)
        y = torch.empty_like(res)
        ops = [
            ("QKV + RoPE", T, (Hq + 2 * Hkv) * D, H,
             lambda: dl.dl_qkv_rope(x, wq, wk, wv, pos, cs, q, k, v),
             (x, wqkv, torch.empty(T, (Hq + 2 * Hkv) * D, dtype=torch.bfloat16, device=dev))),
            ("O", T, H, Hq * D, lambda: dl.dl_linear(attn, wo, o), (attn, wo, o)),
            ("gate/up + SiLU*mul", T, 2 * I, H, lambda: dl.dl_gate_up_silu(x, wg, wu, act),
             (x, wgu, torch.empty(T, 2 * I, dtype=torch.bfloat16, device=dev))),
            ("down + residual", T, H, I, lambda: dl.dl_down_residual(a, wd, y, residual=res),
             (a, wd, o)),
        ]
        for name, M, N, K, ours, (mx, mw, my) in ops:
            fl = 2.0 * M * N * K
            lib_fn = (lambda mx=mx, mw=mw, my=my: torch.mm(mx, mw.t(), out=my))
            t = [cold_ms(ours), _time_ms(ours, n=20), cold_ms(lib_fn), _time_ms(lib_fn, n=20)]
            rows.append((label, name, f"{M} x {N} x {K}",
                         *(f"{ms * 1e3:.1f} us ({fl / ms / 1e9:,.0f})" for ms in t),
                         f"{t[2] / t[0]:.2f}"))
            print(" | ".join(rows[-1]), file=sys.stderr, flush=True)
    lines = ["# Prefill projections: this library against torch.mm (hipBLASLt)", "",
             "Each projection of the 7B layer (2048 tokens) and of the 8B-GQA ragged batch (6235 "
             "tokens) through this library's entry point, with its fused epilogue (RoPE, SiLU*mul, "
             "residual add), and as a plain torch.mm of the same M x N x K (y = x w^T, bf16, no "
             "epilogue).  Cold: 1 GiB written and read before every launch, median of 15 "
             "launches; warm: mean of 20 back-to-back launches.  TFLOP/s in parentheses; the "
             "last column is hipBLASLt's cold time over ours (above 1: ours is faster).", "",
             "Command (repository root on the MI355X box):", "", "```", cmd, "```", "",
             "| workload | projection | M x N x K | ours cold | ours warm | torch.mm cold | "
             "torch.mm warm | torch.mm / ours (cold) |",
             "|---|---|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append("| " + " | ".join(r) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[-len(rows) - 2:]))


def gemm8192(calls: int):
    """The bf16 8192^3 product through this library and through torch.mm
    (hipBLASLt), `calls` times each, for counters."""
    import torch

    from . import binding as dl
    N = 8192
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)
    x = torch.randn(N, N, device="cuda:0", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, N, device="cuda:0", generator=g) * 0.02).to(torch.bfloat16)
    y = torch.empty(N, N, dtype=torch.bfloat16, device="cuda:0")
    torch.cuda.synchronize()
    for _ in range(calls):
        dl.dl_linear(x, w, y)
    for _ in range(calls):
        torch.mm(x, w.t(), out=y)
    torch.cuda.synchronize()
    print(f"ran {calls} products each way", file=sys.stderr)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="sub", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--csv", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="Kernel trace")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--out", required=True)
    c = sub.add_parser("layer-bytes")
    c.add_argument("--mode", choices=["fused", "unfused"], required=True)
    c.add_argument("--calls", type=int, default=3)
    c.add_argument("--config", type=int, choices=[2, 4], default=2)
    e = sub.add_parser("counters")
    e.add_argument("--dirs", nargs="+", required=True)
    e.add_argument("--out", required=True)
    e.add_argument("--cmd", required=True)
    e.add_argument("--title", default="Counters per kernel")
    f_ = sub.add_parser("ceilings")
    f_.add_argument("--out", required=True)
    p_ = sub.add_parser("projections")
    p_.add_argument("--out", required=True)
    g_ = sub.add_parser("gemm8192")
    g_.add_argument("--calls", type=int, default=3)
    d = sub.add_parser("bytes-summary")
    for k in ("fused-fetch", "fused-write", "unfused-fetch", "unfused-write"):
        d.add_argument("--" + k, required=True)
    d.add_argument("--calls", type=int, default=3)
    d.add_argument("--config", type=int, choices=[2, 4], default=2)
    d.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.sub == "stats":
        stats_md(args.csv, args.out, args.cmd, args.title)
    elif args.sub == "traffic":
        t = traffic(args.fetch, args.write)
        with open(args.out, "w") as f:
            json.dump(t, f, indent=1)
        traffic_md(t, os.path.splitext(args.out)[0] + ".md")
        print(json.dumps(t, indent=1))
    elif args.sub == "counters":
        counters_md(args.dirs, args.out, args.cmd, args.title)
    elif args.sub == "ceilings":
        ceilings(args.out, "python -m transformer_decoder_layer_residual_amd.profiling ceilings "
                 f"--out {args.out}")
    elif args.sub == "projections":
        projections(args.out, "python -m transformer_decoder_layer_residual_amd.profiling "
                    f"projections --out {args.out}")
    elif args.sub == "gemm8192":
        gemm8192(args.calls)
    elif args.sub == "layer-bytes":
        run_layer(args.mode, args.calls, args.config)
    else:
        fu = layer_bytes(args.fused_fetch, args.fused_write, args.calls)
        un = layer_bytes(args.unfused_fetch, args.unfused_write, args.calls)
        title = {2: "Llama-2-7B-shaped prefill layer (B1 x 2048)",
                 4: "Llama-3-8B-GQA-shaped prefill layer (8 ragged sequences U{256..1024})"}
        lines = [f"# HBM bytes per {title[args.config]}, fused vs unfused", "",
                 "FETCH_SIZE x 2 + WRITE_SIZE x 1 (copy-kernel calibration), summed over the "
                 "layer's kernels, per layer call.", "",
                 "Commands (repository root on the MI355X box; one counter per run, MODE = fused "
                 "or unfused, COUNTER = FETCH_SIZE or WRITE_SIZE):", "", "```",
                 "cd /tmp && export TMPDIR=/tmp && export PYTHONPATH=$REPO",
                 "rocprofv3 --pmc COUNTER -f csv -d gpurun_out/lb_MODE_COUNTER -o lb -- python -u -m "
                 "transformer_decoder_layer_residual_amd.profiling layer-bytes --mode MODE --calls 3 "
                 f"--config {args.config}",
                 "python -m transformer_decoder_layer_residual_amd.profiling bytes-summary "
                 "--fused-fetch gpurun_out/lb_fused_FETCH_SIZE --fused-write gpurun_out/lb_fused_WRITE_SIZE "
                 "--unfused-fetch gpurun_out/lb_unfused_FETCH_SIZE --unfused-write "
                 f"gpurun_out/lb_unfused_WRITE_SIZE --calls 3 --config {args.config} "
                 "--out profiles/NAME.md", "```", "",
                 "| path | read GB | write GB | total GB |", "|---|---:|---:|---:|",
                 f"| fused | {fu['fetch'] / 1e9:.3f} | {fu['write'] / 1e9:.3f} | {fu['total'] / 1e9:.3f} |",
                 f"| unfused (kernel per op) | {un['fetch'] / 1e9:.3f} | {un['write'] / 1e9:.3f} | "
                 f"{un['total'] / 1e9:.3f} |", "",
                 f"fused / unfused = {fu['total'] / un['total']:.3f}", "", "## per kernel (GB, fused)", ""]
        for k in sorted(fu["fetch_per_kernel"], key=lambda k: -fu["fetch_per_kernel"][k]):
            lines.append(f"- `{k}`: read {fu['fetch_per_kernel'][k] / 1e9:.3f}, write "
                         f"{fu['write_per_kernel'].get(k, 0) / 1e9:.3f}")
        lines += ["", "## per kernel (GB, unfused)", ""]
        for k in sorted(un["fetch_per_kernel"], key=lambda k: -un["fetch_per_kernel"][k]):
            lines.append(f"- `{k}`: read {un['fetch_per_kernel'][k] / 1e9:.3f}, write "
                         f"{un['write_per_kernel'].get(k, 0) / 1e9:.3f}")
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines[:10]))


if __name__ == "__main__":
    main()
