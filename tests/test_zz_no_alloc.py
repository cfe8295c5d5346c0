"""orthros_decode_step_noalloc (the decode step for callers that cannot allocate device memory)
against orthros_decode_step with a workspace: two calls in a row, the second with a smaller
input, each compared with the workspace call on copies of the same state. The two run the same
kernels with the same split count, so the outputs, caches and lengths must agree bit for bit
(which is within the bf16 tolerances of the oracle comparison that the workspace call passes
elsewhere)."""
import pytest
import torch

from efficient_attention_amd import orthros as ox
from efficient_attention_amd import synthetic as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _state(lengths, Hq, Hkv, d, w, seed, cap_extra=4):
    B = len(lengths)
    wl = syn.Workload("noalloc", "decode", B, Hq, Hkv, d, w, "bf16", max(lengths), steps=1,
                      seed=seed)
    inp = syn.make_decode(wl, lengths=lengths)
    cap = max(lengths) + cap_extra
    ck = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    cv = H.nan_like((B, Hkv, cap, d), torch.bfloat16, DEV)
    for b, L in enumerate(lengths):
        ck[b, :, :L] = inp["k"][b, :L].to(DEV).permute(1, 0, 2)
        cv[b, :, :L] = inp["v"][b, :L].to(DEV).permute(1, 0, 2)
    cl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    x = [inp[n][0].to(DEV) for n in ("q_base", "q_out", "k_new", "v_new")]
    shape = ox.Shape(B, Hq, Hkv, d, w, torch.bfloat16, cap)
    return wl, shape, ck, cv, cl, x, H.device_affine(inp["affine"], DEV)


def _compare(lengths, Hq, Hkv, d, w, seed, cap_extra=4, expect_status=0):
    wl, shape, ck, cv, cl, x, aff = _state(lengths, Hq, Hkv, d, w, seed, cap_extra)
    print("[gpu case] no-alloc decode", wl, lengths, flush=True)
    B = shape.batch
    hint = max(lengths)
    outs = {}
    for mode in ("workspace", "noalloc"):
        k2, v2, l2 = ck.clone(), cv.clone(), cl.clone()
        ob = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        oo = H.nan_like((B, Hq, d), torch.bfloat16, DEV)
        if mode == "workspace":
            ws = ox.make_workspace(shape, DEV)
            ox.decode_step(shape, *x, aff, k2, v2, l2, hint, ob, oo, ws)
            status = ox.read_device_status(ws)
        else:
            dst = torch.zeros(1, dtype=torch.int32, device=DEV)
            ox.decode_step_noalloc(shape, *x, aff, k2, v2, l2, hint, ob, oo, dst)
            torch.cuda.synchronize()
            status = int(dst.item())
        torch.cuda.synchronize()
        outs[mode] = (ob, oo, k2, v2, l2, status)
    a, b = outs["workspace"], outs["noalloc"]
    assert not torch.isnan(a[0]).any().item() and not torch.isnan(a[1]).any().item()
    for i, what in enumerate(("o_base", "o_out")):
        assert torch.equal(a[i], b[i]), what
        mx, mr = H.err_stats(H.to64(b[i]), H.to64(a[i]))
        assert mx <= H.BF16_MAX_ABS and mr <= H.BF16_MEAN_REL, what
    for i, what in ((2, "cache_k"), (3, "cache_v")):
        assert torch.equal(a[i].nan_to_num(5.0), b[i].nan_to_num(5.0)), what
    assert torch.equal(a[4], b[4])
    assert a[5] == b[5] == expect_status


def test_noalloc_decode_equals_workspace_decode_twice():
    # first call: 8 sequences of the 8B decode shape, ragged lengths up to 20000 (several splits)
    _compare([20000, 9000, 4097, 131, 64, 1, 15000, 8191], 32, 8, 128, 4096, seed=601)
    # second call, smaller: 2 sequences, fewer heads, d 64; the second sequence's cache is full
    # (capacity = its length), so the step sets the cache-full bit and appends only the first
    _compare([300, 303], 8, 2, 64, 100, seed=602, cap_extra=0, expect_status=ox.STATUS_CACHE_FULL)
