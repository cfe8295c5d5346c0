"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI binding, run the
float64 oracle on host copies of the very same inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from efficient_attention_amd import orthros as ox

# Tolerances. fp32 calls: max-abs 1e-4. bf16 calls: max-abs 1.5e-2 and mean relative error
# (sum |gpu - ref| / sum |ref|) 3e-3, against the oracle on the same bf16-rounded inputs.
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 1.5e-2
BF16_MEAN_REL = 3e-3


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def affine64(aff):
    return tuple(to64(a) for a in aff)


def err_stats(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), "non-finite GPU output (unwritten or overflowed element)"
    diff = np.abs(gpu - ref)
    return float(diff.max()) if diff.size else 0.0, float(diff.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_close(gpu, ref, dtype, what):
    mx, mr = err_stats(gpu, ref)
    if dtype == torch.float32:
        assert mx <= F32_MAX_ABS, f"{what}: max-abs {mx:.3e} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
        assert mr <= BF16_MEAN_REL, f"{what}: mean-rel {mr:.3e} > {BF16_MEAN_REL}"
    return mx, mr


def device_affine(aff, device):
    return ox.Affine(*(a.to(device).contiguous() for a in aff))


def nan_like(shape, dtype, device):
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def gpu_prefill(inp, window, dtype, capacity=None, device="cuda"):
    """Run orthros_prefill on device copies of ``inp`` (from synthetic.make_prefill)."""
    q_base, q_out, k, v = (inp[n].to(device).contiguous() for n in ("q_base", "q_out", "k", "v"))
    B, P, Hq, d = q_base.shape
    Hkv = k.shape[2]
    cap = capacity or P
    shape = ox.Shape(B, Hq, Hkv, d, window, dtype, cap)
    cache_k = nan_like((B, Hkv, cap, d), dtype, device)
    cache_v = nan_like((B, Hkv, cap, d), dtype, device)
    cache_len = torch.full((B,), -7, dtype=torch.int32, device=device)
    o_base = nan_like((B, P, Hq, d), dtype, device)
    o_out = nan_like((B, 1, Hq, d), dtype, device)
    ws = ox.make_workspace(shape, device)
    ox.prefill(shape, q_base, q_out, k, v, device_affine(inp["affine"], device), cache_k, cache_v,
               cache_len, o_base, o_out, ws)
    torch.cuda.synchronize()
    return dict(shape=shape, cache_k=cache_k, cache_v=cache_v, cache_len=cache_len,
                o_base=o_base, o_out=o_out, ws=ws)


def oracle_prefill(inp, window, rows=None):
    return oracle.prefill(to64(inp["q_base"]), to64(inp["q_out"]), to64(inp["k"]), to64(inp["v"]),
                          *affine64(inp["affine"]), window=window, rows=rows)


def cache_as_tokens(cache, length):
    """[B, Hkv, cap, d] head-major cache -> [B, length, Hkv, d] host float64."""
    return to64(cache[:, :, :length].permute(0, 2, 1, 3))
