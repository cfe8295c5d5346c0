"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

The four bf16 workloads run whole on the GPU exactly as the benchmark runs them (same shapes,
capacity, workspace and inputs drawn on the device from the same seeds). The float64 oracle
then evaluates a seeded sample of rows, one at a time, on host copies of the same bf16 values:
edge positions (first keys, the window boundary, the last rows), one row in every block of 64
positions (the prompts) and random ones, every query head. Cache contents are compared bit for
bit in full. The decode workload runs all of its 128 steps; its first and last steps are
compared in full.

Tolerances: max-abs 1.5e-2 and mean relative error 3e-3 over the sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from efficient_attention_amd import orthros as ox
from efficient_attention_amd import synthetic as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[gpu case]", *a, flush=True)


def _positions(T, w, n_random, seed, per_block=False):
    """Edge rows (start, window boundary, tile boundaries, end) plus seeded random rows; with
    per_block, also one seeded row in every block of 64 positions (each block of rows is one
    work-group's share of the banded kernel, so a wrong block-to-rows mapping shows up)."""
    edges = {0, 1, 2, 63, 64, 65, w - 2, w - 1, w, w + 1, T - 65, T - 64, T - 2, T - 1}
    rng = np.random.default_rng(seed)
    pos = edges | set(rng.integers(0, T, size=n_random).tolist())
    if per_block:
        nb = (T + 63) // 64
        pos |= set((64 * np.arange(nb) + rng.integers(0, 64, size=nb)).tolist())
    return sorted(p for p in pos if 0 <= p < T)


def _base_rows_ok(q_rows, K, V, positions, alpha, beta, w, gpu_rows, what):
    """Oracle base rows (Eq. 4) at `positions` against the GPU's rows (all heads)."""
    s = oracle.default_scale(K.shape[-1])
    ref = np.stack([oracle.base_row(oracle.scale_offset(q_rows[i], alpha, beta), K, V, t, w, s)
                    for i, t in enumerate(positions)])
    return H.assert_close(gpu_rows, ref, torch.bfloat16, what)


def _run_prefill_fullsize(name, n_random):
    wl = syn.WORKLOADS[name]
    _say("full-size prefill", wl)
    inp = syn.make_prefill(wl, device=DEV)
    B, P, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, P)
    ck = H.nan_like((B, Hkv, P, d), torch.bfloat16, DEV)
    cv = H.nan_like((B, Hkv, P, d), torch.bfloat16, DEV)
    cl = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ob = H.nan_like((B, P, Hq, d), torch.bfloat16, DEV)
    oo = H.nan_like((B, 1, Hq, d), torch.bfloat16, DEV)
    ws = ox.make_workspace(shape, DEV)
    ox.prefill(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"], ox.Affine(*inp["affine"]),
               ck, cv, cl, ob, oo, ws)
    torch.cuda.synchronize()
    assert cl.cpu().tolist() == [P] * B
    assert torch.equal(ck.permute(0, 2, 1, 3), inp["k"]), "cache_k differs from k"
    assert torch.equal(cv.permute(0, 2, 1, 3), inp["v"]), "cache_v differs from v"
    assert not torch.isnan(ob).any().item(), "unwritten base row"

    a_b, b_b, a_o, b_o = H.affine64(inp["affine"])
    pos = _positions(P, wl.window, n_random, wl.seed, per_block=True)
    idx = torch.as_tensor(pos, device=DEV)
    K = H.to64(inp["k"][0])
    V = H.to64(inp["v"][0])
    q_rows = H.to64(inp["q_base"][0].index_select(0, idx))
    gpu_rows = H.to64(ob[0].index_select(0, idx))
    mb = _base_rows_ok(q_rows, K, V, pos, a_b, b_b, wl.window, gpu_rows, f"{name} o_base")
    s = oracle.default_scale(d)
    ref_out = oracle.output_row(oracle.scale_offset(H.to64(inp["q_out"][0, 0]), a_o, b_o),
                                K, V, P - 1, s)
    mo = H.assert_close(H.to64(oo[0, 0]), ref_out, torch.bfloat16, f"{name} o_out")
    _say(f"{name}: {len(pos)} base rows x {Hq} heads max-abs {mb[0]:.2e} mean-rel {mb[1]:.2e}; "
         f"output row max-abs {mo[0]:.2e} mean-rel {mo[1]:.2e}")
    return wl, inp, K, V, oo


def test_prefill_8b_32k_fullsize():
    _run_prefill_fullsize("prefill_8b_32k", 40)


def test_prefill_8b_128k_planted_fullsize():
    wl, inp, K, V, oo = _run_prefill_fullsize("prefill_8b_128k", 40)
    p = inp["planted_pos"]
    P = wl.length
    assert p is not None and 0 <= p < P - wl.window
    # The planted key is outside every base window that the output row's own position would
    # see, and it dominates the output row of each head h = g G: the oracle's weights put
    # their maximum on it, and the GPU row agrees with the oracle row (checked above).
    G = wl.q_heads // wl.kv_heads
    a_o, b_o = H.to64(inp["affine"][2]), H.to64(inp["affine"][3])
    q_o = oracle.scale_offset(H.to64(inp["q_out"][0, 0]), a_o, b_o)
    s = oracle.default_scale(wl.head_dim)
    for g in range(wl.kv_heads):
        wts = oracle.attention_weights(q_o[g * G], K[:, g, :], s)
        assert int(np.argmax(wts)) == p


def test_pt_1p3b_2k_fullsize():
    wl = syn.WORKLOADS["pt_1p3b_2k"]
    _say("full-size pt", wl)
    inp = syn.make_pt(wl, device=DEV)
    B, T, Hq, d = inp["q_base"].shape
    Hkv = inp["k"].shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, T)
    ob = H.nan_like((B, T, Hq, d), torch.bfloat16, DEV)
    oo = H.nan_like((B, T, Hq, d), torch.bfloat16, DEV)
    ws = ox.make_workspace(shape, DEV)
    ox.forward_pt(shape, inp["q_base"], inp["q_out"], inp["k"], inp["v"],
                  ox.Affine(*inp["affine"]), ob, oo, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(ob).any().item() and not torch.isnan(oo).any().item()
    a_b, b_b, a_o, b_o = H.affine64(inp["affine"])
    s = oracle.default_scale(d)
    worst = [0.0, 0.0]
    for b in range(B):
        pos = _positions(T, wl.window, 12, wl.seed + b)
        idx = torch.as_tensor(pos, device=DEV)
        K = H.to64(inp["k"][b])
        V = H.to64(inp["v"][b])
        mb = _base_rows_ok(H.to64(inp["q_base"][b].index_select(0, idx)), K, V, pos, a_b, b_b,
                           wl.window, H.to64(ob[b].index_select(0, idx)), f"pt o_base b{b}")
        qo = H.to64(inp["q_out"][b].index_select(0, idx))
        ref = np.stack([oracle.output_row(oracle.scale_offset(qo[i], a_o, b_o), K, V, t, s)
                        for i, t in enumerate(pos)])
        mo = H.assert_close(H.to64(oo[b].index_select(0, idx)), ref, torch.bfloat16,
                            f"pt o_out b{b}")
        worst = [max(worst[0], mb[0], mo[0]), max(worst[1], mb[1], mo[1])]
    _say(f"pt_1p3b_2k: max-abs {worst[0]:.2e} mean-rel {worst[1]:.2e}")


def _host64(t: torch.Tensor) -> np.ndarray:
    """Device bf16 -> host float64 (widened to fp32 on the device: exact, and the host side
    only converts fp32 to fp64)."""
    return t.float().cpu().numpy().astype(np.float64)


def test_decode_8b_128k_fullsize():
    """All 128 consecutive steps of the 16 x 131072 decode workload, as the benchmark runs them.

    Every appended cache row of all 16 sequences is compared bit for bit; the first step
    (L = 131072) and the last (L = 131199) are compared, for all 16 sequences, every query head
    and both streams, against the oracle's decode step on that history. Each step draws fresh
    inputs, so one oracle step per checked step is the whole check of that step. The oracle is
    called per kv head (its query heads h = g G .. g G + G - 1 with that kv head's history):
    the same equations, with contiguous host arrays."""
    wl = syn.WORKLOADS["decode_8b_128k"]
    _say("full-size decode, 128 steps", wl)
    S = wl.steps
    B, L0, Hq, Hkv, d = wl.batch, wl.length, wl.q_heads, wl.kv_heads, wl.head_dim
    G = Hq // Hkv
    cap = L0 + wl.steps + 4  # as the benchmark sizes it
    inp = syn.make_decode_resident(wl, DEV, cap)
    ck, cv = inp["cache_k"], inp["cache_v"]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, cap)
    cl = torch.full((B,), L0, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = ox.Affine(*inp["affine"])
    checked = {0: None, S - 1: None}
    for s in range(S):
        ob = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        oo = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        ox.decode_step(shape, inp["q_base"][s], inp["q_out"][s], inp["k_new"][s], inp["v_new"][s],
                       aff, ck, cv, cl, L0 + s, ob, oo, ws)
        if s in checked:
            checked[s] = (ob, oo)
    torch.cuda.synchronize()
    _say("128 steps done")
    assert cl.cpu().tolist() == [L0 + S] * B
    assert ox.read_device_status(ws) == 0
    # every appended row of every sequence, bit for bit
    assert torch.equal(ck[:, :, L0:L0 + S], inp["k_new"].permute(1, 2, 0, 3))
    assert torch.equal(cv[:, :, L0:L0 + S], inp["v_new"].permute(1, 2, 0, 3))
    a64 = H.affine64(inp["affine"])
    ref = {s: (np.empty((B, Hq, d)), np.empty((B, Hq, d))) for s in checked}
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            cs = slice(g * G * d, (g + 1) * G * d)
            # this kv head's history through the last checked step (keys 0 .. L0 + S - 2);
            # the oracle reads its first L rows for a step at length L
            Kg = _host64(ck[b, g, :L0 + S - 1])[:, None, :]
            Vg = _host64(cv[b, g, :L0 + S - 1])[:, None, :]
            for s in checked:
                r = oracle.decode_step(
                    [Kg], [Vg], np.array([L0 + s]), H.to64(inp["q_base"][s, b:b + 1, hs]),
                    H.to64(inp["q_out"][s, b:b + 1, hs]),
                    H.to64(inp["k_new"][s, b:b + 1, g:g + 1]),
                    H.to64(inp["v_new"][s, b:b + 1, g:g + 1]), a64[0][cs], a64[1][cs],
                    a64[2][cs], a64[3][cs], window=wl.window)
                ref[s][0][b, hs], ref[s][1][b, hs] = r[0][0], r[1][0]
        _say(f"oracle: sequence {b} done")
    for s, (ob, oo) in checked.items():
        assert not torch.isnan(ob).any().item() and not torch.isnan(oo).any().item()
        mb = H.assert_close(H.to64(ob), ref[s][0], torch.bfloat16, f"o_base step {s}")
        mo = H.assert_close(H.to64(oo), ref[s][1], torch.bfloat16, f"o_out step {s}")
        _say(f"decode step {s} (L = {L0 + s}), 16 sequences x 32 heads: base max-abs "
             f"{mb[0]:.2e} rel {mb[1]:.2e}; out max-abs {mo[0]:.2e} rel {mo[1]:.2e}")


def test_decode_8b_128k_paged_equals_contiguous():
    """The full-size decode workload with its history dealt into a shuffled pool of 64-token
    pages: two steps, outputs bit for bit equal to the contiguous cache's (same kernels and
    arithmetic; test_decode_8b_128k_fullsize checks those against the oracle)."""
    wl = syn.WORKLOADS["decode_8b_128k"]
    _say("full-size paged decode", wl)
    B, L0, Hq, Hkv, d = wl.batch, wl.length, wl.q_heads, wl.kv_heads, wl.head_dim
    ps = 64
    max_pages = -(-(L0 + wl.steps + 4) // ps)
    cap = max_pages * ps
    inp = syn.make_decode_resident(wl, DEV, cap)
    ck, cv = inp["cache_k"], inp["cache_v"]
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 11)
    num_pages = B * max_pages
    table = torch.randperm(num_pages, generator=g, device=DEV).view(B, max_pages)
    kp = torch.empty(num_pages, Hkv, ps, d, dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    nb = L0 // ps
    for b in range(B):
        idx = table[b, :nb]
        kp[idx] = ck[b, :, :L0].reshape(Hkv, nb, ps, d).permute(1, 0, 2, 3)
        vp[idx] = cv[b, :, :L0].reshape(Hkv, nb, ps, d).permute(1, 0, 2, 3)
    cache = ox.PagedKV(kp, vp, table.to(torch.int32).contiguous())
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, torch.bfloat16, cap)
    cl_c = torch.full((B,), L0, dtype=torch.int32, device=DEV)
    cl_p = cl_c.clone()
    ws_c, ws_p = ox.make_workspace(shape, DEV), ox.make_workspace(shape, DEV)
    aff = ox.Affine(*inp["affine"])
    for s in range(2):
        args = [inp[n][s] for n in ("q_base", "q_out", "k_new", "v_new")]
        outs = [torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
        ox.decode_step(shape, *args, aff, ck, cv, cl_c, L0 + s, outs[0], outs[1], ws_c)
        ox.decode_step_paged(shape, *args, aff, cache, cl_p, L0 + s, outs[2], outs[3], ws_p)
        torch.cuda.synchronize()
        assert not torch.isnan(outs[0]).any().item()
        assert torch.equal(outs[0], outs[2]), f"o_base differs at step {s}"
        assert torch.equal(outs[1], outs[3]), f"o_out differs at step {s}"
    assert torch.equal(cl_c, cl_p)
    assert ox.read_device_status(ws_p) == 0
    for s in range(2):
        t = L0 + s
        page = table[:, t // ps]
        assert torch.equal(kp[page, :, t % ps], inp["k_new"][s])
        assert torch.equal(vp[page, :, t % ps], inp["v_new"][s])


def test_pt_1p3b_2k_training_fullsize():
    """Pre-training forward (with lse) and backward at the 1.3B shape (4 x 2048 tokens, 16 heads,
    d 128, window 512) in the launch configuration the benchmark times; every element of every
    gradient against the float64 oracle on the same inputs (drawn on the device)."""
    from tests.test_gpu_training import check_against_oracle, run_training
    wl = syn.WORKLOADS["pt_1p3b_2k"]
    _say("full-size training", wl)
    inp, do_b, do_o, got = run_training(wl, device=DEV)
    inp = {n: (t.cpu() if isinstance(t, torch.Tensor) else
               tuple(a.cpu() for a in t) if isinstance(t, tuple) else t) for n, t in inp.items()}
    worst = check_against_oracle(wl, inp, do_b.cpu(), do_o.cpu(), got)
    _say("pt_1p3b_2k training: " + " ".join(f"{n} {m[1]:.2e}" for n, m in worst.items()))
