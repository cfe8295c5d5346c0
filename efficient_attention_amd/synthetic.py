"""Seeded synthetic inputs for the Orthros attention workloads.

This module only draws random numbers and shapes them; it holds none of the attention
arithmetic, so both the HIP path's tests/benchmark and the float64 oracle consume exactly the
tensors it returns (the oracle gets host float64 copies of the same values).

Recipes (the pages print no inputs; these are the documented stand-ins):
  * every q/k/v entry ~ N(0, 1), drawn in float32 from a seeded ``torch.Generator`` in a fixed
    order (q_base, q_out, k, v, then the scale-offset vectors), then rounded once to the
    storage dtype (round-to-nearest-even for bf16);
  * scale-offset vectors (the paper's alpha, beta, alpha', beta', §3.1): scale
    1 + 0.1 N(0, 1) and offset 0.1 N(0, 1), float32, one entry per (query head, channel),
    drawn separately for the base and the output stream;
  * ``rms_norm``: each (b, t, head) row of q_base, q_out, k, v is divided by its root mean
    square before rounding;
  * ``planted``: for every KV head g, the key row at a seeded position p in [0, P - w) is
    replaced by the raw output-stream query of head g*G (a copy of input values), so a
    retrieval target sits far outside every base row's window but inside the output row's
    full history (a stand-in for a long-context needle test);
  * decode: each step draws fresh q_base, q_out, k_new, v_new (no model feedback).

Random draws happen on ``device`` (CPU for small cases; the GPU's generator for the large
ones, where host generation would dominate the run time). The stream differs between
devices, so a record always names the device its inputs were drawn on.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_affine", "make_prefill", "make_pt", "make_decode",
           "make_decode_resident", "make_sft", "bf16_round"]


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "prefill" | "pt" | "decode" | "sft"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    dtype: str                # "f32" | "bf16"
    length: int               # prompt length P (prefill), T (pt/sft), cache length L0 (decode)
    steps: int = 0            # decode steps
    rms_norm: bool = False
    planted: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 sequence, 1 head, d 64, prompt 256, window 32, fp32, one output row at the end.
    "tiny_fp32_prefill": Workload("tiny_fp32_prefill", "prefill", 1, 1, 1, 64, 32, "f32",
                                  256, seed=1),
    # Pre-training regime at a 1.3B-like attention shape: batch 4, T 2048, 16 heads MHA.
    "pt_1p3b_2k": Workload("pt_1p3b_2k", "pt", 4, 16, 16, 128, 512, "bf16", 2048,
                           rms_norm=True, seed=2),
    # Llama3.1-8B attention shape, prompt 32768, GQA 32/8, window 4096.
    "prefill_8b_32k": Workload("prefill_8b_32k", "prefill", 1, 32, 8, 128, 4096, "bf16",
                               32768, seed=3),
    # Same shape at 131072 with one planted high-similarity key per KV head.
    "prefill_8b_128k": Workload("prefill_8b_128k", "prefill", 1, 32, 8, 128, 4096, "bf16",
                                131072, planted=True, seed=4),
    # 16 sequences holding 131072-token caches, 128 decode steps.
    "decode_8b_128k": Workload("decode_8b_128k", "decode", 16, 32, 8, 128, 4096, "bf16",
                               131072, steps=128, seed=5),
}


def _dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to bfloat16 (round-to-nearest-even), returned as bfloat16."""
    return x.to(torch.bfloat16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, rms_norm=False):
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if rms_norm:
        x = x / x.pow(2).mean(dim=-1, keepdim=True).sqrt()
    return x


def make_affine(q_heads: int, head_dim: int, g: torch.Generator, device):
    """Scale-offset vectors [H_q * d] float32: (alpha_b, beta_b, alpha_o, beta_o)."""
    n = q_heads * head_dim
    out = []
    for _ in range(2):
        a = 1.0 + 0.1 * torch.randn(n, generator=g, device=device, dtype=torch.float32)
        b = 0.1 * torch.randn(n, generator=g, device=device, dtype=torch.float32)
        out += [a, b]
    return tuple(out)


def make_prefill(w: Workload, device="cpu"):
    """Prefill inputs: q_base [B,P,Hq,d], q_out [B,1,Hq,d], k, v [B,P,Hkv,d], affine."""
    g = _gen(w.seed, device)
    B, P, Hq, Hkv, d = w.batch, w.length, w.q_heads, w.kv_heads, w.head_dim
    dt = _dtype(w.dtype)
    q_base = _normal((B, P, Hq, d), g, device, w.rms_norm).to(dt)
    q_out = _normal((B, 1, Hq, d), g, device, w.rms_norm).to(dt)
    k = _normal((B, P, Hkv, d), g, device, w.rms_norm).to(dt)
    v = _normal((B, P, Hkv, d), g, device, w.rms_norm).to(dt)
    aff = make_affine(Hq, d, g, device)
    planted_pos = None
    if w.planted:
        span = max(1, P - w.window)
        planted_pos = int(torch.randint(0, span, (1,), generator=g, device=device).item())
        G = Hq // Hkv
        for kv in range(Hkv):
            k[:, planted_pos, kv, :] = q_out[:, 0, kv * G, :]
    return dict(q_base=q_base, q_out=q_out, k=k, v=v, affine=aff, planted_pos=planted_pos)


def make_pt(w: Workload, device="cpu"):
    """Pre-training inputs: q_base, q_out [B,T,Hq,d], k, v [B,T,Hkv,d], affine."""
    g = _gen(w.seed, device)
    B, T, Hq, Hkv, d = w.batch, w.length, w.q_heads, w.kv_heads, w.head_dim
    dt = _dtype(w.dtype)
    q_base = _normal((B, T, Hq, d), g, device, w.rms_norm).to(dt)
    q_out = _normal((B, T, Hq, d), g, device, w.rms_norm).to(dt)
    k = _normal((B, T, Hkv, d), g, device, w.rms_norm).to(dt)
    v = _normal((B, T, Hkv, d), g, device, w.rms_norm).to(dt)
    aff = make_affine(Hq, d, g, device)
    return dict(q_base=q_base, q_out=q_out, k=k, v=v, affine=aff)


def make_sft(w: Workload, out_positions, device="cpu"):
    """SFT inputs: like pre-training, but q_out holds only the rows at ``out_positions``."""
    d = make_pt(w, device)
    g = _gen(w.seed + 7919, device)
    B, Hq = w.batch, w.q_heads
    d["q_out"] = _normal((B, len(out_positions), Hq, w.head_dim), g, device,
                         w.rms_norm).to(_dtype(w.dtype))
    d["out_positions"] = list(out_positions)
    return d


def make_decode(w: Workload, device="cpu", lengths=None):
    """Decode inputs.

    Returns prefix k, v [B, L0, Hkv, d] (the history each sequence already holds), per-step
    q_base, q_out [S, B, Hq, d], k_new, v_new [S, B, Hkv, d], the affine vectors and the
    per-sequence starting lengths (``lengths`` or L0 for all).
    """
    g = _gen(w.seed, device)
    B, L0, S, Hq, Hkv, d = w.batch, w.length, w.steps, w.q_heads, w.kv_heads, w.head_dim
    dt = _dtype(w.dtype)
    k = _normal((B, L0, Hkv, d), g, device).to(dt)
    v = _normal((B, L0, Hkv, d), g, device).to(dt)
    q_base = _normal((S, B, Hq, d), g, device).to(dt)
    q_out = _normal((S, B, Hq, d), g, device).to(dt)
    k_new = _normal((S, B, Hkv, d), g, device).to(dt)
    v_new = _normal((S, B, Hkv, d), g, device).to(dt)
    aff = make_affine(Hq, d, g, device)
    lens = [L0] * B if lengths is None else list(lengths)
    return dict(k=k, v=v, q_base=q_base, q_out=q_out, k_new=k_new, v_new=v_new, affine=aff,
                lengths=lens)


def make_decode_resident(w: Workload, device, capacity: int):
    """Decode inputs drawn straight into a device-resident head-major cache.

    For the full-size decode workload (16 x 131072 tokens) a token-major prefix plus a copy
    would double the 8.6 GB footprint, so the history is drawn per sequence into
    cache_k, cache_v [B, H_kv, capacity, d] (rows 0..L0-1; the rest left unset), in the order
    k then v for each sequence, each ~ N(0, 1) rounded once to the storage dtype. Then the
    per-step q_base, q_out [S, B, H_q, d], k_new, v_new [S, B, H_kv, d] and the affine vectors.
    """
    g = _gen(w.seed, device)
    B, L0, S, Hq, Hkv, d = w.batch, w.length, w.steps, w.q_heads, w.kv_heads, w.head_dim
    dt = _dtype(w.dtype)
    ck = torch.empty(B, Hkv, capacity, d, dtype=dt, device=device)
    cv = torch.empty_like(ck)
    for t in (ck, cv):
        for b in range(B):
            t[b, :, :L0].copy_(torch.randn(Hkv, L0, d, generator=g, device=device))
    q_base = _normal((S, B, Hq, d), g, device).to(dt)
    q_out = _normal((S, B, Hq, d), g, device).to(dt)
    k_new = _normal((S, B, Hkv, d), g, device).to(dt)
    v_new = _normal((S, B, Hkv, d), g, device).to(dt)
    aff = make_affine(Hq, d, g, device)
    return dict(cache_k=ck, cache_v=cv, q_base=q_base, q_out=q_out, k_new=k_new, v_new=v_new,
                affine=aff, lengths=[L0] * B)
