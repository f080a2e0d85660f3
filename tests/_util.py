"""Shared helpers for the GPU parity tests: host<->device moves and the
tolerance rules used against the oracle.

Tolerance (bf16 storage, fp32 accumulation; the oracle in its bf16-storage
mode is fed the GPU's own bf16 inputs):
  * bf16 tensors: relative L2 error <= 1e-2, and per element
    |gpu - ref| <= max(3e-2, one bf16 ulp of ref) (a different summation
    order may flip one rounding boundary);
  * fp32 residual-stream outputs: relative L2 <= 1e-2 and max |diff| <= 3e-2;
  * integer / copy work: bit-exact.
"""
import numpy as np
import torch

import oracle

DEV = "cuda:0"


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(a):
    return dev_f32(a).to(torch.bfloat16)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_as(a, dtype):
    return dev_bf16(a) if dtype == torch.bfloat16 else dev_f32(a)


def dev_cache(bits):
    """uint16 (bf16 bits) or uint32 (fp32 bits) host cache -> device tensor."""
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(bits.view(np.float32)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy()


def host_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float32))
    e = np.floor(np.log2(np.maximum(x, np.float32(1e-38))))
    return np.exp2(e - 7).astype(np.float32)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def assert_bf16_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    r = rel_l2(gpu, ref)
    assert r <= 1e-2, f"{what}: rel-L2 {r:.3e}"
    bound = np.maximum(np.float32(3e-2), bf16_ulp(ref))
    bad = np.abs(gpu - ref) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond max(3e-2, 1 ulp); "
                           f"worst {np.abs(gpu - ref).max():.4g}")
    return r


def assert_f32_close(gpu, ref, what="", max_abs=3e-2, rel=1e-2):
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    r = rel_l2(gpu, ref)
    m = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
    assert r <= rel, f"{what}: rel-L2 {r:.3e}"
    assert m <= max_abs, f"{what}: max-abs {m:.3e}"
    return r, m


def bf(a):
    return oracle.bf16_round(np.asarray(a, np.float32))
