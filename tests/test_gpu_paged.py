"""GPU parity for decoding over a paged key/value cache and for the paged bulk write.

The pool's pages are dealt to the sequences in a seeded random order, and every slot that no
sequence owns holds NaN, so a read from a wrong page or slot shows up as a non-finite output.
Outputs are compared with the float64 oracle (decode_step_paged / paged_write) element by
element, pools and lengths bit for bit, and the paged path with the contiguous one bit for bit
(same kernels and arithmetic; only the row addresses differ)."""
import math

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


def _pool(hists, ps, max_pages, Hkv, d, tdt, seed, spare=3):
    """Pages of a shuffled pool filled from per-sequence histories [L_b, H_kv, d] (host);
    unowned slots are NaN. Returns (k_pages, v_pages, table) on the device."""
    B = len(hists)
    num_pages = B * max_pages + spare
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages)
    pools = []
    for which in range(2):
        pool = torch.full((num_pages, Hkv, ps, d), float("nan"), dtype=tdt)
        for b, hv in enumerate(hists):
            h = hv[which]
            for i in range(math.ceil(h.shape[0] / ps)):
                blk = h[i * ps:(i + 1) * ps]
                pool[table[b, i], :, :blk.shape[0]] = blk.permute(1, 0, 2)
        pools.append(pool.to(DEV))
    return pools[0], pools[1], table.to(torch.int32).to(DEV)


CASES = [
    # (Hq, Hkv, d, w, page size, lengths, dtype)
    (8, 2, 128, 100, 64, [300, 129, 64], "bf16"),
    (4, 1, 128, 33, 16, [77, 200], "bf16"),
    (4, 2, 64, 8, 1, [50, 3], "bf16"),
    (32, 8, 128, 4096, 256, [5000], "bf16"),
    (8, 2, 128, 64, 128, [0, 130], "bf16"),      # an empty sequence
    (4, 2, 64, 20, 32, [45, 90], "f32"),
]


@pytest.mark.parametrize("Hq,Hkv,d,w,ps,lengths,dt", CASES)
def test_paged_decode_matches_oracle(Hq, Hkv, d, w, ps, lengths, dt):
    steps = 3
    B = len(lengths)
    wl = syn.Workload("paged", "decode", B, Hq, Hkv, d, w, dt, max(lengths), steps=steps,
                      seed=900 + ps + sum(lengths))
    _say("paged decode", wl, "page", ps, lengths)
    inp = syn.make_decode(wl, lengths=lengths)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    max_pages = math.ceil((max(lengths) + steps) / ps) + 1
    cap = max_pages * ps
    hists = [(inp["k"][b, :lengths[b]], inp["v"][b, :lengths[b]]) for b in range(B)]
    kp, vp, table = _pool(hists, ps, max_pages, Hkv, d, tdt, wl.seed)
    cache = ox.PagedKV(kp, vp, table)
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, cap)
    cl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    a64 = H.affine64(inp["affine"])
    rk, rv, lens, tbl = H.to64(kp), H.to64(vp), np.array(lengths), table.cpu().numpy()
    for s in range(steps):
        ob = H.nan_like((B, Hq, d), tdt, DEV)
        oo = H.nan_like((B, Hq, d), tdt, DEV)
        ox.decode_step_paged(shape, inp["q_base"][s].to(DEV), inp["q_out"][s].to(DEV),
                             inp["k_new"][s].to(DEV), inp["v_new"][s].to(DEV), aff, cache, cl,
                             int(lens.max()), ob, oo, ws)
        torch.cuda.synchronize()
        rb, ro, rk, rv, lens, full = oracle.decode_step_paged(
            rk, rv, tbl, lens, H.to64(inp["q_base"][s]), H.to64(inp["q_out"][s]),
            H.to64(inp["k_new"][s]), H.to64(inp["v_new"][s]), *a64, window=w)
        assert not full.any()
        H.assert_close(H.to64(ob), rb, tdt, f"o_base step {s}")
        H.assert_close(H.to64(oo), ro, tdt, f"o_out step {s}")
    assert cl.cpu().tolist() == lens.tolist()
    np.testing.assert_array_equal(H.to64(kp), rk)
    np.testing.assert_array_equal(H.to64(vp), rv)
    assert ox.read_device_status(ws) == 0


@pytest.mark.parametrize("ps", [64, 16])
def test_paged_decode_equals_contiguous_decode_bitwise(ps):
    B, Hq, Hkv, d, w = 4, 32, 8, 128, 4096
    lengths = [9000, 5000, 12000, 700]
    wl = syn.Workload("paged_vs_contig", "decode", B, Hq, Hkv, d, w, "bf16", max(lengths),
                      steps=2, seed=950 + ps)
    _say("paged == contiguous", wl, "page", ps)
    inp = syn.make_decode(wl, lengths=lengths)
    max_pages = math.ceil((max(lengths) + 2) / ps)
    cap = max_pages * ps
    shape = ox.Shape(B, Hq, Hkv, d, w, torch.bfloat16, cap)
    ck = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    cv = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    for b, L in enumerate(lengths):
        ck[b, :, :L] = inp["k"][b, :L].to(DEV).permute(1, 0, 2)
        cv[b, :, :L] = inp["v"][b, :L].to(DEV).permute(1, 0, 2)
    hists = [(inp["k"][b, :lengths[b]], inp["v"][b, :lengths[b]]) for b in range(B)]
    kp, vp, table = _pool(hists, ps, max_pages, Hkv, d, torch.bfloat16, wl.seed)
    cache = ox.PagedKV(kp, vp, table)
    cl_c = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    cl_p = cl_c.clone()
    ws_c, ws_p = ox.make_workspace(shape, DEV), ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    for s in range(2):
        args = [inp[n][s].to(DEV) for n in ("q_base", "q_out", "k_new", "v_new")]
        outs = [torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
        ox.decode_step(shape, *args, aff, ck, cv, cl_c, max(lengths) + s, outs[0], outs[1], ws_c)
        ox.decode_step_paged(shape, *args, aff, cache, cl_p, max(lengths) + s, outs[2], outs[3],
                             ws_p)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[2]), f"o_base differs at step {s}"
        assert torch.equal(outs[1], outs[3]), f"o_out differs at step {s}"
    assert torch.equal(cl_c, cl_p)
    for b, L in enumerate(lengths):  # the two appended rows, read back through the table
        for t in (L, L + 1):
            page, slot = int(table[b, t // ps]), t % ps
            assert torch.equal(kp[page, :, slot], ck[b, :, t])
            assert torch.equal(vp[page, :, slot], cv[b, :, t])
    assert ox.read_device_status(ws_p) == 0


def test_paged_write_matches_oracle_and_reports_full():
    B, Hkv, d, ps, max_pages, T = 4, 2, 128, 16, 16, 50  # capacity 256
    starts = [0, 37, 200, 230]                             # the last has no room for 50 more
    g = torch.Generator().manual_seed(31)
    k = torch.randn(B, T, Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, T, Hkv, d, generator=g).to(torch.bfloat16)
    _say("paged write", B, T, ps, starts)
    num_pages = B * max_pages + 2
    table = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages)
    kp = torch.randn(num_pages, Hkv, ps, d, generator=g).to(torch.bfloat16).to(DEV)
    vp = torch.randn(num_pages, Hkv, ps, d, generator=g).to(torch.bfloat16).to(DEV)
    rk0, rv0 = H.to64(kp), H.to64(vp)
    table = table.to(torch.int32).to(DEV)
    shape = ox.Shape(B, 4, Hkv, d, 8, torch.bfloat16, max_pages * ps)
    cl = torch.tensor(starts, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    ox.paged_write(shape, k.to(DEV), v.to(DEV), ox.PagedKV(kp, vp, table), cl, ws)
    torch.cuda.synchronize()
    rk, rv, lens, full = oracle.paged_write(rk0, rv0, table.cpu().numpy(), np.array(starts),
                                            H.to64(k), H.to64(v))
    assert full.tolist() == [False, False, False, True]
    assert cl.cpu().tolist() == lens.tolist()
    np.testing.assert_array_equal(H.to64(kp), rk)
    np.testing.assert_array_equal(H.to64(vp), rv)
    assert ox.read_device_status(ws, clear=True) == ox.STATUS_CACHE_FULL


def test_paged_prompt_write_then_decode_matches_oracle():
    """A prompt written into pages by the bulk write, then decode steps over it."""
    B, Hq, Hkv, d, w, ps, P, steps = 2, 8, 2, 128, 48, 32, 150, 3
    wl = syn.Workload("paged_flow", "decode", B, Hq, Hkv, d, w, "bf16", P, steps=steps, seed=77)
    _say("paged prompt + decode", wl)
    inp = syn.make_decode(wl)
    max_pages = math.ceil((P + steps) / ps) + 1
    num_pages = B * max_pages + 1
    g = torch.Generator().manual_seed(78)
    table = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages)
    table = table.to(torch.int32).to(DEV)
    kp = torch.full((num_pages, Hkv, ps, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    cache = ox.PagedKV(kp, vp, table)
    shape = ox.Shape(B, Hq, Hkv, d, w, torch.bfloat16, max_pages * ps)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    ox.paged_write(shape, inp["k"].to(DEV), inp["v"].to(DEV), cache, cl, ws)
    aff = H.device_affine(inp["affine"], DEV)
    rk, rv, lens, _ = oracle.paged_write(H.to64(kp), H.to64(vp), table.cpu().numpy(),
                                         np.zeros(B, dtype=np.int64), H.to64(inp["k"]),
                                         H.to64(inp["v"]))
    tbl = table.cpu().numpy()
    for s in range(steps):
        ob = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        oo = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        ox.decode_step_paged(shape, inp["q_base"][s].to(DEV), inp["q_out"][s].to(DEV),
                             inp["k_new"][s].to(DEV), inp["v_new"][s].to(DEV), aff, cache, cl,
                             P + s, ob, oo, ws)
        torch.cuda.synchronize()
        rb, ro, rk, rv, lens, _ = oracle.decode_step_paged(
            rk, rv, tbl, lens, H.to64(inp["q_base"][s]), H.to64(inp["q_out"][s]),
            H.to64(inp["k_new"][s]), H.to64(inp["v_new"][s]), *H.affine64(inp["affine"]),
            window=w)
        H.assert_close(H.to64(ob), rb, torch.bfloat16, f"o_base step {s}")
        H.assert_close(H.to64(oo), ro, torch.bfloat16, f"o_out step {s}")
    assert cl.cpu().tolist() == lens.tolist() == [P + steps] * B
    np.testing.assert_array_equal(H.to64(kp), rk)
    assert ox.read_device_status(ws) == 0


def test_paged_decode_full_and_bad_page_status():
    """Sequence 0 is full (not appended, outputs still exact); sequence 1's table names a page
    outside the pool for the block of its new token (flagged, nothing written, length kept);
    sequence 2 is ordinary and stays exact."""
    B, Hq, Hkv, d, w, ps, max_pages = 3, 4, 2, 128, 16, 16, 4  # capacity 64
    lengths = [64, 40, 20]
    wl = syn.Workload("paged_status", "decode", B, Hq, Hkv, d, w, "bf16", 64, steps=1, seed=88)
    _say("paged status", wl)
    inp = syn.make_decode(wl, lengths=lengths)
    hists = [(inp["k"][b, :lengths[b]], inp["v"][b, :lengths[b]]) for b in range(B)]
    kp, vp, table = _pool(hists, ps, max_pages, Hkv, d, torch.bfloat16, wl.seed)
    num_pages = kp.shape[0]
    table[1, 40 // ps] = num_pages  # position 40's block: not a page of the pool
    kp_before = kp.clone()
    shape = ox.Shape(B, Hq, Hkv, d, w, torch.bfloat16, max_pages * ps)
    cl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    ob = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV)
    oo = torch.empty_like(ob)
    ox.decode_step_paged(shape, inp["q_base"][0].to(DEV), inp["q_out"][0].to(DEV),
                         inp["k_new"][0].to(DEV), inp["v_new"][0].to(DEV),
                         H.device_affine(inp["affine"], DEV), ox.PagedKV(kp, vp, table), cl, 64,
                         ob, oo, ws)
    torch.cuda.synchronize()
    st = ox.read_device_status(ws, clear=True)
    assert st == ox.STATUS_CACHE_FULL | ox.STATUS_BAD_PAGE
    assert cl.cpu().tolist() == [64, 40, 21]
    rb, ro, _, _, _ = oracle.decode_step(
        [H.to64(h[0]) for h in hists], [H.to64(h[1]) for h in hists], np.array(lengths),
        H.to64(inp["q_base"][0]), H.to64(inp["q_out"][0]), H.to64(inp["k_new"][0]),
        H.to64(inp["v_new"][0]), *H.affine64(inp["affine"]), window=w)
    for b in (0, 2):
        H.assert_close(H.to64(ob[b]), rb[b], torch.bfloat16, f"o_base seq {b}")
        H.assert_close(H.to64(oo[b]), ro[b], torch.bfloat16, f"o_out seq {b}")
    # only sequence 2's new row was written
    changed = (kp != kp_before) & ~(torch.isnan(kp) & torch.isnan(kp_before))
    slots = torch.nonzero(changed.any(dim=3).any(dim=1)).tolist()  # [page, slot] pairs
    assert slots == [[int(table[2, 20 // ps]), 20 % ps]]


PREFILL_CASES = [
    # (B, Hq, Hkv, d, page size, chunks, w, dtype)
    (2, 8, 2, 128, 64, [100, 37, 200], 64, "bf16"),   # windows reach back across chunks
    (1, 4, 4, 128, 128, [130, 130], 300, "bf16"),     # window longer than everything
    (1, 4, 2, 64, 64, [65, 64, 63], 65, "bf16"),       # d 64, tile-boundary chunk sizes
    (2, 4, 2, 64, 16, [40, 33], 20, "f32"),            # fp32 rows take any page size
]


# last_only: the chunks before the last pass no output row (q_out = o_out = None).
@pytest.mark.parametrize("B,Hq,Hkv,d,ps,chunks,w,dt,last_only",
                         [c + (False,) for c in PREFILL_CASES] + [PREFILL_CASES[0] + (True,)])
def test_paged_prefill_in_chunks_then_decode_matches_oracle(B, Hq, Hkv, d, ps, chunks, w, dt,
                                                            last_only):
    P = sum(chunks)
    steps = 2
    wl = syn.Workload("paged_chunks", "prefill", B, Hq, Hkv, d, w, dt, P, seed=1100 + P + ps)
    _say("paged prefill chunks", wl, chunks, "page", ps, "last only" if last_only else "")
    inp = syn.make_prefill(wl)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    max_pages = math.ceil((P + steps) / ps) + 1
    num_pages = B * max_pages + 2
    g = torch.Generator().manual_seed(wl.seed + 3)
    table = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages)
    table = table.to(torch.int32).to(DEV)
    kp = torch.full((num_pages, Hkv, ps, d), float("nan"), dtype=tdt, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    cache = ox.PagedKV(kp, vp, table)
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, max_pages * ps)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    a64 = H.affine64(inp["affine"])
    tbl = table.cpu().numpy()
    rk, rv = H.to64(kp), H.to64(vp)
    hk = np.zeros((B, 0, Hkv, d))
    hv = np.zeros((B, 0, Hkv, d))
    past = 0
    for c in chunks:
        sl = slice(past, past + c)
        qo = torch.randn(B, 1, Hq, d, generator=g).to(tdt)
        ob = H.nan_like((B, c, Hq, d), tdt, DEV)
        oo = H.nan_like((B, 1, Hq, d), tdt, DEV)
        kc, vc = inp["k"][:, sl].contiguous(), inp["v"][:, sl].contiguous()
        row = not last_only or past + c == P  # this chunk computes the output row
        ox.prefill_chunk_paged(shape, past, inp["q_base"][:, sl].contiguous().to(DEV),
                               qo.to(DEV) if row else None, kc.to(DEV), vc.to(DEV), aff, cache,
                               cl, ob, oo if row else None, ws)
        torch.cuda.synchronize()
        rb, ro, hk, hv, _ = oracle.prefill_chunk(hk, hv, past, H.to64(inp["q_base"][:, sl]),
                                                 H.to64(qo), H.to64(kc), H.to64(vc), *a64,
                                                 window=w)
        rk, rv, lens, _ = oracle.paged_write(rk, rv, tbl, np.full(B, past), H.to64(kc),
                                             H.to64(vc))
        H.assert_close(H.to64(ob), rb, tdt, f"o_base chunk at {past}")
        if row:
            H.assert_close(H.to64(oo), ro, tdt, f"o_out chunk at {past}")
        past += c
        assert cl.cpu().tolist() == lens.tolist() == [past] * B
    np.testing.assert_array_equal(H.to64(kp), rk)
    np.testing.assert_array_equal(H.to64(vp), rv)
    lens = np.full(B, P)
    for s in range(steps):
        x = [torch.randn(B, Hq, d, generator=g).to(tdt) for _ in range(2)]
        x += [torch.randn(B, Hkv, d, generator=g).to(tdt) for _ in range(2)]
        ob = H.nan_like((B, Hq, d), tdt, DEV)
        oo = H.nan_like((B, Hq, d), tdt, DEV)
        ox.decode_step_paged(shape, *(t.to(DEV) for t in x), aff, cache, cl, P + s, ob, oo, ws)
        torch.cuda.synchronize()
        rb, ro, rk, rv, lens, _ = oracle.decode_step_paged(rk, rv, tbl, lens,
                                                           *(H.to64(t) for t in x), *a64,
                                                           window=w)
        H.assert_close(H.to64(ob), rb, tdt, f"decode o_base step {s}")
        H.assert_close(H.to64(oo), ro, tdt, f"decode o_out step {s}")
    np.testing.assert_array_equal(H.to64(kp), rk)
    assert ox.read_device_status(ws) == 0
