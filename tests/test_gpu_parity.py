"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same inputs.

Small cases compare every output element; they span several 64-key tiles, ragged tails,
windows of 1, w-1, w, w+1 and >= T, grouped and plain multi-head attention, d 64 and 128.
Each test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle
from efficient_attention_amd import orthros as ox
from efficient_attention_amd import synthetic as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(**kw):
    base = dict(name="case", mode="prefill", batch=1, q_heads=4, kv_heads=1, head_dim=128,
                window=64, dtype="bf16", length=200, seed=11)
    base.update(kw)
    return syn.Workload(**base)


def _say(*a):
    print("[gpu case]", *a, flush=True)


# --------------------------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------------------------
def test_tiny_fp32_prefill_workload():
    w = syn.WORKLOADS["tiny_fp32_prefill"]
    _say(w)
    inp = syn.make_prefill(w)
    g = H.gpu_prefill(inp, w.window, torch.float32)
    ob, oo, ck, cv, ln = H.oracle_prefill(inp, w.window)
    H.assert_close(H.to64(g["o_base"]), ob, torch.float32, "o_base")
    H.assert_close(H.to64(g["o_out"]), oo, torch.float32, "o_out")
    np.testing.assert_array_equal(H.cache_as_tokens(g["cache_k"], w.length), ck)
    np.testing.assert_array_equal(H.cache_as_tokens(g["cache_v"], w.length), cv)
    assert g["cache_len"].cpu().tolist() == ln.tolist()


PREFILL_CASES = [
    # (batch, Hq, Hkv, d, P, window, dtype)
    (1, 4, 1, 128, 200, 64, "bf16"),     # GQA 4, ragged tail, window = one tile
    (2, 8, 2, 128, 333, 100, "bf16"),    # window not a tile multiple
    (1, 2, 2, 128, 130, 1, "bf16"),      # window 1 returns V
    (1, 4, 4, 128, 257, 300, "bf16"),    # window >= P: plain causal
    (1, 8, 1, 128, 96, 63, "bf16"),      # GQA 8
    (1, 4, 2, 64, 190, 65, "bf16"),      # d 64
    (1, 3, 1, 128, 70, 31, "bf16"),      # odd group size
    (1, 16, 1, 128, 77, 40, "bf16"),     # group 16 (two head chunks per kv head)
    (1, 1, 1, 128, 1, 5, "bf16"),        # single token
    (2, 4, 2, 64, 150, 7, "f32"),        # fp32 path
    (1, 2, 1, 128, 129, 128, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,P,w,dt", PREFILL_CASES)
def test_prefill_matches_oracle(B, Hq, Hkv, d, P, w, dt):
    wl = _case(batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=d, length=P, window=w, dtype=dt,
               seed=100 + P)
    _say("prefill", wl)
    inp = syn.make_prefill(wl)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = H.gpu_prefill(inp, w, tdt, capacity=P + 5)
    ob, oo, ck, cv, ln = H.oracle_prefill(inp, w)
    H.assert_close(H.to64(g["o_base"]), ob, tdt, "o_base")
    H.assert_close(H.to64(g["o_out"]), oo, tdt, "o_out")
    np.testing.assert_array_equal(H.cache_as_tokens(g["cache_k"], P), ck)
    np.testing.assert_array_equal(H.cache_as_tokens(g["cache_v"], P), cv)
    assert g["cache_len"].cpu().tolist() == [P] * B
    # rows past the prompt stay untouched
    assert torch.isnan(g["cache_k"][:, :, P:].float()).all()


def _far_key_inputs(wl, amp):
    """Prefill inputs with one key far below the rows that see it: key 50 gets the direction u
    scaled by amp, and the base queries of rows 400..649 (after their scale-offset) the same, so
    their score against it is amp^2 s log2 e (log2 units), while their scores against the keys
    near their diagonal stay of the order of amp."""
    inp = syn.make_prefill(wl)
    g = torch.Generator().manual_seed(wl.seed + 1)
    u = torch.randn(wl.head_dim, generator=g, dtype=torch.float64)
    u /= u.norm()
    a_b, b_b = (x.double().view(wl.q_heads, wl.head_dim) for x in inp["affine"][:2])
    inp["k"][0, 50, 0, :] = (amp * u).to(inp["k"].dtype)
    for t in range(400, 650):
        inp["q_base"][0, t] = ((amp * u[None, :] - b_b) / a_b).to(inp["q_base"].dtype)
    return inp


def test_prefill_far_dominant_key_matches_oracle():
    """A key that dominates rows far above it (as a sink token does): rows 400..649 meet it more
    than 300 keys below their diagonal, with a score 80-90 (log2 units) above every score they
    met before it. The band kernel's reference then moves by that much in one rescale (the
    accumulated output scaled by ~2^-85), and the rows' weight sits on that key."""
    wl = _case(batch=1, q_heads=4, kv_heads=1, head_dim=128, length=700, window=600,
               dtype="bf16", seed=4242)
    inp = _far_key_inputs(wl, 27.3)
    _say("prefill, far dominant key", wl)
    s = oracle.default_scale(wl.head_dim) * np.log2(np.e)
    q64 = oracle.scale_offset(H.to64(inp["q_base"][0]), *H.affine64(inp["affine"][:2]))
    k64 = H.to64(inp["k"][0, :, 0])
    for t in (400, 500, 649):  # the jump the rows meet, from the scores of the pages' Eq. 4
        sc = q64[t] @ k64[: t + 1].T * s  # [Hq, t + 1], log2 units
        jump = sc[:, 50] - sc[:, t - 300:].max(axis=1)
        assert ((jump > 60) & (jump < 110)).all(), jump
    g = H.gpu_prefill(inp, wl.window, torch.bfloat16)
    ob, oo, _, _, _ = H.oracle_prefill(inp, wl.window)
    H.assert_close(H.to64(g["o_base"]), ob, torch.bfloat16, "o_base")
    H.assert_close(H.to64(g["o_out"]), oo, torch.bfloat16, "o_out")
    v50 = H.to64(inp["v"][0, 50, 0])
    np.testing.assert_allclose(H.to64(g["o_base"][0, 500]), np.broadcast_to(v50, (4, 128)),
                               atol=2e-2)


def test_prefill_cache_is_ready_on_the_callers_stream():
    """Work enqueued after the call on the caller's own stream (here a non-default one, not
    synchronised in between) already sees the whole cache and cache_len."""
    wl = _case(batch=2, q_heads=8, kv_heads=2, head_dim=128, length=1000, window=200,
               dtype="bf16", seed=321)
    _say("prefill on a side stream", wl)
    inp = syn.make_prefill(wl)
    tdt = torch.bfloat16
    q_base, q_out, k, v = (inp[n].to(DEV).contiguous() for n in ("q_base", "q_out", "k", "v"))
    B, P, Hq, d = q_base.shape
    Hkv = k.shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, tdt, P)
    cache_k = H.nan_like((B, Hkv, P, d), tdt, DEV)
    cache_v = H.nan_like((B, Hkv, P, d), tdt, DEV)
    cache_len = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    o_base = H.nan_like((B, P, Hq, d), tdt, DEV)
    o_out = H.nan_like((B, 1, Hq, d), tdt, DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        ox.prefill(shape, q_base, q_out, k, v, aff, cache_k, cache_v, cache_len, o_base, o_out,
                   ws, stream=st)
        ck = cache_k.clone()
        cv = cache_v.clone()
        ln = cache_len.clone()
    torch.cuda.synchronize()
    _, _, rk, rv, _ = H.oracle_prefill(inp, wl.window)
    np.testing.assert_array_equal(H.cache_as_tokens(ck, P), rk)
    np.testing.assert_array_equal(H.cache_as_tokens(cv, P), rv)
    assert ln.cpu().tolist() == [P] * B


def test_prefill_is_deterministic():
    wl = _case(batch=1, q_heads=8, kv_heads=2, length=700, window=256, seed=5)
    _say("determinism", wl)
    inp = syn.make_prefill(wl)
    a = H.gpu_prefill(inp, wl.window, torch.bfloat16)
    b = H.gpu_prefill(inp, wl.window, torch.bfloat16)
    assert torch.equal(a["o_base"], b["o_base"]) and torch.equal(a["o_out"], b["o_out"])


# --------------------------------------------------------------------------------------------
# Pre-training regime
# --------------------------------------------------------------------------------------------
PT_CASES = [
    (2, 4, 4, 128, 300, 64, "bf16"),
    (1, 8, 2, 128, 257, 100, "bf16"),
    (1, 4, 1, 64, 130, 200, "bf16"),
    (1, 2, 1, 64, 100, 9, "f32"),
]


def _gpu_pt(inp, window, tdt, with_cache=False):
    q_base, q_out, k, v = (inp[n].to(DEV).contiguous() for n in ("q_base", "q_out", "k", "v"))
    B, T, Hq, d = q_base.shape
    Hkv = k.shape[2]
    shape = ox.Shape(B, Hq, Hkv, d, window, tdt, T)
    ob = H.nan_like((B, T, Hq, d), tdt, DEV)
    oo = H.nan_like((B, T, Hq, d), tdt, DEV)
    ws = ox.make_workspace(shape, DEV)
    kw = {}
    if with_cache:
        kw = dict(cache_k=H.nan_like((B, Hkv, T, d), tdt, DEV),
                  cache_v=H.nan_like((B, Hkv, T, d), tdt, DEV),
                  cache_len=torch.zeros(B, dtype=torch.int32, device=DEV))
    ox.forward_pt(shape, q_base, q_out, k, v, H.device_affine(inp["affine"], DEV), ob, oo, ws, **kw)
    torch.cuda.synchronize()
    return ob, oo, kw


@pytest.mark.parametrize("B,Hq,Hkv,d,T,w,dt", PT_CASES)
def test_pt_matches_oracle(B, Hq, Hkv, d, T, w, dt):
    wl = _case(mode="pt", batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=d, length=T, window=w,
               dtype=dt, seed=200 + T, rms_norm=True)
    _say("pt", wl)
    inp = syn.make_pt(wl)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ob, oo, kw = _gpu_pt(inp, w, tdt, with_cache=True)
    rb, ro = oracle.forward_pt(H.to64(inp["q_base"]), H.to64(inp["q_out"]), H.to64(inp["k"]),
                               H.to64(inp["v"]), *H.affine64(inp["affine"]), window=w)
    H.assert_close(H.to64(ob), rb, tdt, "o_base")
    H.assert_close(H.to64(oo), ro, tdt, "o_out")
    np.testing.assert_array_equal(H.cache_as_tokens(kw["cache_k"], T), H.to64(inp["k"]))
    assert kw["cache_len"].cpu().tolist() == [T] * B


# --------------------------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------------------------
def _decode_run(wl, steps, lengths, tdt, capacity):
    """Fill caches with the synthetic prefix, run `steps` decode steps, compare every step."""
    inp = syn.make_decode(wl.scaled(steps=steps), lengths=lengths)
    B, L0, Hkv, d = inp["k"].shape
    Hq = wl.q_heads
    shape = ox.Shape(B, Hq, Hkv, d, wl.window, tdt, capacity)
    ck = H.nan_like((B, Hkv, capacity, d), tdt, DEV)
    cv = H.nan_like((B, Hkv, capacity, d), tdt, DEV)
    ck[:, :, :L0] = inp["k"].to(DEV).permute(0, 2, 1, 3)
    cv[:, :, :L0] = inp["v"].to(DEV).permute(0, 2, 1, 3)
    cl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    hist_k = [H.to64(inp["k"][b, :lengths[b]]) for b in range(B)]
    hist_v = [H.to64(inp["v"][b, :lengths[b]]) for b in range(B)]
    lens = np.array(lengths)
    for s in range(steps):
        ob = H.nan_like((B, Hq, d), tdt, DEV)
        oo = H.nan_like((B, Hq, d), tdt, DEV)
        ox.decode_step(shape, inp["q_base"][s].to(DEV), inp["q_out"][s].to(DEV),
                       inp["k_new"][s].to(DEV), inp["v_new"][s].to(DEV), aff, ck, cv, cl,
                       int(lens.max()), ob, oo, ws)
        torch.cuda.synchronize()
        rb, ro, hist_k, hist_v, lens = oracle.decode_step(
            hist_k, hist_v, lens, H.to64(inp["q_base"][s]), H.to64(inp["q_out"][s]),
            H.to64(inp["k_new"][s]), H.to64(inp["v_new"][s]), *H.affine64(inp["affine"]),
            window=wl.window)
        H.assert_close(H.to64(ob), rb, tdt, f"o_base step {s}")
        H.assert_close(H.to64(oo), ro, tdt, f"o_out step {s}")
    assert cl.cpu().tolist() == lens.tolist()
    for b in range(B):
        np.testing.assert_array_equal(H.to64(ck[b, :, :lens[b]].permute(1, 0, 2)), hist_k[b])
        np.testing.assert_array_equal(H.to64(cv[b, :, :lens[b]].permute(1, 0, 2)), hist_v[b])
    return ws, ck, cl


@pytest.mark.parametrize("Hq,Hkv,d,w,lengths,dt", [
    (8, 2, 128, 64, [300, 5, 64, 1000], "bf16"),
    (8, 2, 128, 50, [0, 63, 127, 128], "bf16"),  # empty history; new key at a tile's end / start
    (4, 4, 128, 1, [77, 200], "bf16"),
    (32, 8, 128, 4096, [5000, 9000], "bf16"),
    (16, 1, 64, 100, [150], "bf16"),
    (4, 2, 64, 30, [40, 90], "f32"),
])
def test_decode_matches_oracle(Hq, Hkv, d, w, lengths, dt):
    wl = _case(mode="decode", batch=len(lengths), q_heads=Hq, kv_heads=Hkv, head_dim=d,
               window=w, dtype=dt, length=max(lengths), seed=300 + w)
    _say("decode", wl, lengths)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ws, _, _ = _decode_run(wl, 3, lengths, tdt, capacity=max(lengths) + 8)
    assert ox.read_device_status(ws) == 0


def test_decode_cache_full_sets_status_and_keeps_outputs_exact():
    wl = _case(mode="decode", batch=2, q_heads=4, kv_heads=2, window=16, length=40, seed=9)
    _say("decode cache full", wl)
    # capacity 41: sequence 0 (len 40) appends once, then is full; sequence 1 has room.
    inp = syn.make_decode(wl.scaled(steps=2), lengths=[40, 10])
    B, L0, Hkv, d = inp["k"].shape
    cap = 41
    shape = ox.Shape(B, 4, Hkv, d, 16, torch.bfloat16, cap)
    ck = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    cv = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    ck[:, :, :L0] = inp["k"].to(DEV).permute(0, 2, 1, 3)
    cv[:, :, :L0] = inp["v"].to(DEV).permute(0, 2, 1, 3)
    cl = torch.tensor([40, 10], dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    hk = [H.to64(inp["k"][0, :40]), H.to64(inp["k"][1, :10])]
    hv = [H.to64(inp["v"][0, :40]), H.to64(inp["v"][1, :10])]
    lens = np.array([40, 10])
    for s in range(2):
        ob = H.nan_like((B, 4, d), torch.bfloat16, DEV)
        oo = H.nan_like((B, 4, d), torch.bfloat16, DEV)
        ox.decode_step(shape, inp["q_base"][s].to(DEV), inp["q_out"][s].to(DEV),
                       inp["k_new"][s].to(DEV), inp["v_new"][s].to(DEV), aff, ck, cv, cl, 41,
                       ob, oo, ws)
        torch.cuda.synchronize()
        rb, ro, nk, nv, nl = oracle.decode_step(
            hk, hv, lens, H.to64(inp["q_base"][s]), H.to64(inp["q_out"][s]),
            H.to64(inp["k_new"][s]), H.to64(inp["v_new"][s]), *H.affine64(inp["affine"]), window=16)
        H.assert_close(H.to64(ob), rb, torch.bfloat16, "o_base")
        H.assert_close(H.to64(oo), ro, torch.bfloat16, "o_out")
        # the library keeps what fits: a full sequence is not extended
        for b in range(B):
            if lens[b] < cap:
                hk[b], hv[b], lens[b] = nk[b], nv[b], nl[b]
    assert cl.cpu().tolist() == [41, 12]
    assert ox.read_device_status(ws, clear=True) == ox.STATUS_CACHE_FULL
    assert ox.read_device_status(ws) == 0


def test_pt_equals_prefill_then_decode_on_gpu():
    """§3.2 consistency on the GPU itself: batch PT rows equal prefill + decode steps."""
    wl = _case(mode="pt", batch=2, q_heads=8, kv_heads=2, length=160, window=48, seed=77)
    _say("pt vs incremental", wl)
    inp = syn.make_pt(wl)
    ob, oo, _ = _gpu_pt(inp, wl.window, torch.bfloat16)
    P0 = 150
    pre = dict(q_base=inp["q_base"][:, :P0], q_out=inp["q_out"][:, P0 - 1:P0],
               k=inp["k"][:, :P0], v=inp["v"][:, :P0], affine=inp["affine"])
    g = H.gpu_prefill(pre, wl.window, torch.bfloat16, capacity=wl.length)
    worst = 0.0
    worst = max(worst, H.err_stats(H.to64(g["o_base"]), H.to64(ob[:, :P0]))[0])
    worst = max(worst, H.err_stats(H.to64(g["o_out"][:, 0]), H.to64(oo[:, P0 - 1]))[0])
    aff = H.device_affine(inp["affine"], DEV)
    for t in range(P0, wl.length):
        db = H.nan_like((2, 8, 128), torch.bfloat16, DEV)
        do = H.nan_like((2, 8, 128), torch.bfloat16, DEV)
        ox.decode_step(g["shape"], inp["q_base"][:, t].contiguous().to(DEV),
                       inp["q_out"][:, t].contiguous().to(DEV), inp["k"][:, t].contiguous().to(DEV),
                       inp["v"][:, t].contiguous().to(DEV), aff, g["cache_k"], g["cache_v"],
                       g["cache_len"], t, db, do, g["ws"])
        torch.cuda.synchronize()
        worst = max(worst, H.err_stats(H.to64(db), H.to64(ob[:, t]))[0])
        worst = max(worst, H.err_stats(H.to64(do), H.to64(oo[:, t]))[0])
    # both sides round to bf16 independently: a few bf16 ulps of the outputs at most
    assert worst <= 1.5e-2, worst
