"""Seeded randomized small-shape sweep of the HIP path against the float64 oracle.

A fixed seed draws a fixed list of cases over the grid the edge cases of "Orthros: Phase-Aware
Heterogeneous Attention for Efficient Transformers" §3.1 Eq. 4/5 live on: prompt lengths
T in {1, 2, w-1, w, w+1, an odd length}, windows w in {1, 2, 31, 64, >= T}, query heads per
kv head G in {1, 2, 4, 8}, head_dim in {64, 128}, fp32 and bf16, one or two sequences and one
or two kv heads. Each case runs prefill (every base row, the output row at the last token, the
cache) followed by one decode step, and the pre-training forward on the same inputs, every
output element compared with the oracle. The list is fixed, so a failure names a case that
reruns the same way (run with -x to stop at the first one)."""
import numpy as np
import pytest
import torch

import oracle
from efficient_attention_amd import orthros as ox
from efficient_attention_amd import synthetic as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 40


def _draw_cases(seed=20261202, n=N_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        w_kind = rng.integers(0, 5)
        w = [1, 2, 31, 64, None][w_kind]
        base_T = int(rng.integers(3, 200))
        if w is None:  # window at least the prompt: plain causal rows
            w = base_T + int(rng.integers(0, 50))
        T = [1, 2, max(1, w - 1), w, w + 1, 2 * int(rng.integers(1, 150)) + 1][rng.integers(0, 6)]
        G = int([1, 2, 4, 8][rng.integers(0, 4)])
        Hkv = int(rng.integers(1, 3))
        d = int([64, 128][rng.integers(0, 2)])
        dt = ["f32", "bf16"][rng.integers(0, 2)]
        B = int(rng.integers(1, 3))
        cases.append((i, B, G * Hkv, Hkv, d, int(T), int(w), dt))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("i,B,Hq,Hkv,d,T,w,dt", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_case_matches_oracle(i, B, Hq, Hkv, d, T, w, dt):
    wl = syn.Workload(f"sweep{i}", "pt", B, Hq, Hkv, d, w, dt, T, seed=7000 + i)
    print("[gpu case] sweep", wl, flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp = syn.make_pt(wl)
    a64 = H.affine64(inp["affine"])
    # prefill of the T-token prompt (output query: the last row of q_out), capacity T + 1
    pre = dict(q_base=inp["q_base"], q_out=inp["q_out"][:, T - 1:T].contiguous(), k=inp["k"],
               v=inp["v"], affine=inp["affine"])
    g = H.gpu_prefill(pre, w, tdt, capacity=T + 1)
    rb, ro, rk, rv, rl = H.oracle_prefill(pre, w)
    H.assert_close(H.to64(g["o_base"]), rb, tdt, "prefill o_base")
    H.assert_close(H.to64(g["o_out"]), ro, tdt, "prefill o_out")
    np.testing.assert_array_equal(H.cache_as_tokens(g["cache_k"], T), rk)
    assert g["cache_len"].cpu().tolist() == [T] * B
    # one decode step after it
    gen = torch.Generator().manual_seed(8000 + i)
    x = [torch.randn(B, Hq, d, generator=gen).to(tdt) for _ in range(2)]
    x += [torch.randn(B, Hkv, d, generator=gen).to(tdt) for _ in range(2)]
    db = H.nan_like((B, Hq, d), tdt, DEV)
    do = H.nan_like((B, Hq, d), tdt, DEV)
    ox.decode_step(g["shape"], *(t.to(DEV) for t in x), H.device_affine(inp["affine"], DEV),
                   g["cache_k"], g["cache_v"], g["cache_len"], T, db, do, g["ws"])
    torch.cuda.synchronize()
    sb, so, _, _, sl = oracle.decode_step(list(rk), list(rv), rl, *(H.to64(t) for t in x), *a64,
                                          window=w)
    H.assert_close(H.to64(db), sb, tdt, "decode o_base")
    H.assert_close(H.to64(do), so, tdt, "decode o_out")
    assert g["cache_len"].cpu().tolist() == sl.tolist()
    assert ox.read_device_status(g["ws"]) == 0
    # the pre-training forward on the same inputs
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, T)
    ob = H.nan_like((B, T, Hq, d), tdt, DEV)
    oo = H.nan_like((B, T, Hq, d), tdt, DEV)
    ox.forward_pt(shape, *(inp[n].to(DEV) for n in ("q_base", "q_out", "k", "v")),
                  H.device_affine(inp["affine"], DEV), ob, oo, ox.make_workspace(shape, DEV))
    torch.cuda.synchronize()
    pb, po = oracle.forward_pt(*(H.to64(inp[n]) for n in ("q_base", "q_out", "k", "v")), *a64,
                               window=w)
    H.assert_close(H.to64(ob), pb, tdt, "pt o_base")
    H.assert_close(H.to64(oo), po, tdt, "pt o_out")
