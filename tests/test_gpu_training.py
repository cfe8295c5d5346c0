"""GPU parity of the training path: the pre-training forward with per-row log-sum-exp, and the
backward pass of both streams (raw queries, keys, values, scale-offset vectors), against the
float64 oracle on the same inputs, every element.

Tolerances: outputs as for the forward; lse max-abs 2e-2 (bf16) / 1e-4 (fp32). Gradients in
fp32: max-abs 1e-4. bf16 gradients: mean relative error 5e-3 and max-abs 1e-2 x the tensor's
largest magnitude. Each bf16 gradient passes through up to four bf16 roundings (the
post-affine query, the probabilities for dv, the score gradient for dq and dk, and the rounded
forward output inside D = rowsum(dO O)), each worth up to 2^-9 relative; the forward's outputs,
with two, sit at about 2.5e-3."""
import numpy as np
import pytest
import torch

import oracle
from efficient_attention_amd import orthros as ox
from efficient_attention_amd import synthetic as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRAD_MEAN_REL = 5e-3
GRAD_MAX_FRAC = 1e-2


def _say(*a):
    print("[gpu case]", *a, flush=True)


def _grad_close(gpu, ref, dtype, what):
    mx, mr = H.err_stats(gpu, ref)
    if dtype == torch.float32:
        assert mx <= H.F32_MAX_ABS, f"{what}: max-abs {mx:.3e}"
    else:
        scale = float(np.abs(ref).max())
        assert mx <= GRAD_MAX_FRAC * max(scale, 1e-30), f"{what}: max-abs {mx:.3e} vs {scale:.3e}"
        assert mr <= GRAD_MEAN_REL, f"{what}: mean-rel {mr:.3e}"
    return mx, mr


def run_training(wl, device=DEV, seed_do=None):
    """Forward (with lse) and backward on the GPU; returns host copies and the inputs."""
    inp = syn.make_pt(wl, device=device)
    B, T, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    tdt = inp["q_base"].dtype
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + 101 if seed_do is None else seed_do)
    do_b = torch.randn(B, T, Hq, d, generator=g, device=device).to(tdt)
    do_o = torch.randn(B, T, Hq, d, generator=g, device=device).to(tdt)
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, tdt, T)
    q_base, q_out, k, v = (inp[n].to(DEV).contiguous() for n in ("q_base", "q_out", "k", "v"))
    aff = H.device_affine(inp["affine"], DEV)
    ob = H.nan_like((B, T, Hq, d), tdt, DEV)
    oo = H.nan_like((B, T, Hq, d), tdt, DEV)
    lb = H.nan_like((B, Hq, T), torch.float32, DEV)
    lo = H.nan_like((B, Hq, T), torch.float32, DEV)
    ws = ox.make_workspace(shape, DEV)
    ox.forward_pt_lse(shape, q_base, q_out, k, v, aff, ob, oo, lb, lo, ws)
    bws = torch.empty(ox.backward_workspace_bytes(shape, T), dtype=torch.uint8, device=DEV)
    dqb, dqo = H.nan_like((B, T, Hq, d), tdt, DEV), H.nan_like((B, T, Hq, d), tdt, DEV)
    dk, dv = H.nan_like((B, T, Hkv, d), tdt, DEV), H.nan_like((B, T, Hkv, d), tdt, DEV)
    dg = [H.nan_like((Hq * d,), torch.float32, DEV) for _ in range(4)]
    ox.backward_pt(shape, q_base, q_out, k, v, aff, ob, oo, lb, lo, do_b.to(DEV), do_o.to(DEV),
                   dqb, dqo, dk, dv, dg, bws)
    torch.cuda.synchronize()
    gpu = dict(o_base=ob, o_out=oo, lse_base=lb, lse_out=lo, dq_base=dqb, dq_out=dqo, dk=dk,
               dv=dv, dalpha_b=dg[0], dbeta_b=dg[1], dalpha_o=dg[2], dbeta_o=dg[3])
    return inp, do_b, do_o, {n: H.to64(t) for n, t in gpu.items()}


def check_against_oracle(wl, inp, do_b, do_o, got):
    tdt = inp["q_base"].dtype
    a64 = H.affine64(inp["affine"])
    q_b, q_o, k, v = (H.to64(inp[n]) for n in ("q_base", "q_out", "k", "v"))
    rb, ro = oracle.forward_pt(q_b, q_o, k, v, *a64, window=wl.window)
    H.assert_close(got["o_base"], rb, tdt, "o_base")
    H.assert_close(got["o_out"], ro, tdt, "o_out")
    rlb, rlo = oracle.lse_pt(q_b, q_o, k, *a64, window=wl.window)
    lse_tol = 1e-4 if tdt == torch.float32 else 2e-2
    for n, r in (("lse_base", rlb), ("lse_out", rlo)):
        mx, _ = H.err_stats(got[n], r)
        assert mx <= lse_tol, f"{n}: max-abs {mx:.3e}"
    gr = oracle.backward_pt(q_b, q_o, k, v, *a64, H.to64(do_b), H.to64(do_o), window=wl.window)
    worst = {}
    for n in ("dq_base", "dq_out", "dk", "dv", "dalpha_b", "dbeta_b", "dalpha_o", "dbeta_o"):
        if not np.abs(gr[n]).max() > 0:  # window 1: the base stream's query gradients vanish
            assert np.abs(got[n]).max() <= 1e-5, n
            continue
        worst[n] = _grad_close(got[n], gr[n], tdt, n)
    return worst


CASES = [
    # (B, Hq, Hkv, d, T, w, dtype)
    (1, 4, 2, 64, 150, 40, "f32"),
    (2, 4, 1, 128, 200, 64, "bf16"),
    (1, 8, 2, 128, 333, 100, "bf16"),     # ragged tail, GQA 4
    (1, 4, 4, 64, 130, 1, "bf16"),        # window 1: base rows are v, query gradients zero
    (1, 4, 2, 128, 96, 500, "bf16"),      # window longer than the sequence
    (1, 2, 1, 128, 1, 8, "bf16"),         # one token
    (2, 4, 2, 64, 70, 33, "f32"),
    (3, 7, 7, 64, 512, 100, "bf16"),      # 21 (sequence, head) pairs: the causal and key-side
                                          # work orders end on a partial group of pairs
    (1, 16, 2, 128, 320, 128, "bf16"),    # eight query heads per kv head (8-wavefront groups)
]


@pytest.mark.parametrize("B,Hq,Hkv,d,T,w,dt", CASES)
def test_training_forward_and_backward_match_oracle(B, Hq, Hkv, d, T, w, dt):
    wl = syn.Workload("train", "pt", B, Hq, Hkv, d, w, dt, T, seed=700 + T + w)
    _say("training", wl)
    inp, do_b, do_o, got = run_training(wl, device="cpu")
    worst = check_against_oracle(wl, inp, do_b, do_o, got)
    _say(" ".join(f"{n} {m[1]:.2e}" for n, m in worst.items()))


def test_backward_is_deterministic():
    wl = syn.Workload("train_det", "pt", 1, 8, 2, 128, 64, "bf16", 300, seed=42)
    _say("determinism", wl)
    a = run_training(wl, device="cpu")[3]
    b = run_training(wl, device="cpu")[3]
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


SFT_CASES = [
    # (B, Hq, Hkv, d, T, w, positions, dtype)
    (2, 4, 2, 128, 200, 64, list(range(150, 200)), "bf16"),                       # suffix
    (1, 8, 2, 128, 300, 100, [5, 299, 150, 151, 0, 64, 63, 200, 201, 202], "bf16"),  # unsorted
    (1, 4, 1, 64, 130, 17, [129], "bf16"),                                        # one row
    (1, 4, 2, 128, 96, 40, [10, 10, 50, 95, 95, 30] * 7, "bf16"),                 # R > 32, repeats
    (1, 4, 2, 64, 90, 20, [89, 3, 45, 46, 47], "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,T,w,pos,dt", SFT_CASES)
def test_sft_training_matches_oracle(B, Hq, Hkv, d, T, w, pos, dt):
    wl = syn.Workload("sft_train", "sft", B, Hq, Hkv, d, w, dt, T, seed=800 + T + len(pos))
    _say("sft training", wl, "rows", len(pos))
    inp = syn.make_sft(wl, pos)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    R = len(pos)
    g = torch.Generator().manual_seed(wl.seed + 5)
    do_b = torch.randn(B, T, Hq, d, generator=g).to(tdt)
    do_o = torch.randn(B, R, Hq, d, generator=g).to(tdt)
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, T)
    q_base, q_out, k, v = (inp[n].to(DEV).contiguous() for n in ("q_base", "q_out", "k", "v"))
    aff = H.device_affine(inp["affine"], DEV)
    op = torch.tensor(pos, dtype=torch.int32, device=DEV)
    ob, oo = H.nan_like((B, T, Hq, d), tdt, DEV), H.nan_like((B, R, Hq, d), tdt, DEV)
    lb, lo = H.nan_like((B, Hq, T), torch.float32, DEV), H.nan_like((B, Hq, R), torch.float32, DEV)
    ws = ox.make_workspace(shape, DEV, sft_rows=R)
    ox.forward_sft_lse(shape, q_base, q_out, op, k, v, aff, ob, oo, lb, lo, ws)
    bws = torch.empty(ox.backward_sft_workspace_bytes(shape, T, R), dtype=torch.uint8, device=DEV)
    dqb, dqo = H.nan_like((B, T, Hq, d), tdt, DEV), H.nan_like((B, R, Hq, d), tdt, DEV)
    dk, dv = H.nan_like((B, T, Hkv, d), tdt, DEV), H.nan_like((B, T, Hkv, d), tdt, DEV)
    dg = [H.nan_like((Hq * d,), torch.float32, DEV) for _ in range(4)]
    ox.backward_sft(shape, q_base, q_out, op, k, v, aff, ob, oo, lb, lo, do_b.to(DEV),
                    do_o.to(DEV), dqb, dqo, dk, dv, dg, bws)
    torch.cuda.synchronize()
    a64 = H.affine64(inp["affine"])
    x = [H.to64(inp[n]) for n in ("q_base", "q_out", "k", "v")]
    rb, ro = oracle.forward_sft(*x, pos, *a64, window=w)
    H.assert_close(H.to64(ob), rb, tdt, "o_base")
    H.assert_close(H.to64(oo), ro, tdt, "o_out")
    rlb, rlo = oracle.lse_sft(x[0], x[1], x[2], pos, *a64, window=w)
    lse_tol = 1e-4 if tdt == torch.float32 else 2e-2
    for got, r, n in ((lb, rlb, "lse_base"), (lo, rlo, "lse_out")):
        assert H.err_stats(H.to64(got), r)[0] <= lse_tol, n
    gr = oracle.backward_sft(*x, pos, *a64, H.to64(do_b), H.to64(do_o), window=w)
    got = dict(dq_base=dqb, dq_out=dqo, dk=dk, dv=dv, dalpha_b=dg[0], dbeta_b=dg[1],
               dalpha_o=dg[2], dbeta_o=dg[3])
    for n, t in got.items():
        _grad_close(H.to64(t), gr[n], tdt, n)
