"""GPU parity for the supervised fine-tuning regime and for prefill in chunks.

SFT (orthros_forward_sft): base rows everywhere, output rows at given response positions; up
to 16 response rows run on the split-key kernel, more on the banded kernel with a row list
(unsorted positions included). Chunked prefill (orthros_prefill_chunk): a prompt fed in
pieces whose windows reach back into the cached tokens of earlier pieces. Every output element
is compared with the float64 oracle on the same inputs; caches bit for bit."""
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


def _wl(**kw):
    base = dict(name="case", mode="sft", batch=1, q_heads=4, kv_heads=1, head_dim=128,
                window=64, dtype="bf16", length=200, seed=21)
    base.update(kw)
    return syn.Workload(**base)


SFT_CASES = [
    # (B, Hq, Hkv, d, T, w, positions, dtype, with_cache)
    (2, 8, 2, 128, 300, 64, [5, 150, 299], "bf16", False),              # split rows
    (1, 4, 1, 128, 257, 31, [0], "bf16", True),                          # single row at 0
    (1, 8, 2, 128, 400, 100, list(range(384, 400)), "bf16", False),      # 16 rows: split limit
    (1, 4, 2, 64, 333, 65, [100, 3, 332, 64, 65], "bf16", False),        # d 64, unsorted
    (2, 4, 1, 128, 500, 50, list(range(420, 500)), "bf16", True),        # 80 rows: banded path
    (1, 8, 2, 128, 260, 40, [259, 7, 130, 64, 63, 200, 1, 0, 255, 128, 129, 30, 31, 32, 33,
                             100, 101, 102, 250, 251], "bf16", False),  # 20 unsorted: banded
    (1, 4, 4, 64, 200, 33, list(range(150, 200)), "bf16", True),         # d 64, MHA, 50 rows
    (2, 16, 2, 128, 180, 48, [179, 0, 90, 91, 17, 179, 60, 120, 5, 6, 7, 8, 150, 151, 33, 34,
                              100, 101, 170, 2, 44, 45, 46, 47], "bf16", False),  # 8 heads/kv, 24
    (1, 4, 2, 64, 150, 9, [149, 0, 77], "f32", False),                  # fp32 rows
    (1, 4, 2, 128, 129, 128, list(range(100, 129)), "f32", False),      # fp32, 29 rows
]


@pytest.mark.parametrize("B,Hq,Hkv,d,T,w,pos,dt,with_cache", SFT_CASES)
def test_sft_matches_oracle(B, Hq, Hkv, d, T, w, pos, dt, with_cache):
    wl = _wl(batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=d, length=T, window=w, dtype=dt,
             seed=400 + T + len(pos))
    _say("sft", wl, "rows", len(pos))
    inp = syn.make_sft(wl, pos)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    R = len(pos)
    q_base, q_out, k, v = (inp[n].to(DEV).contiguous() for n in ("q_base", "q_out", "k", "v"))
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, T)
    ob = H.nan_like((B, T, Hq, d), tdt, DEV)
    oo = H.nan_like((B, R, Hq, d), tdt, DEV)
    ws = ox.make_workspace(shape, DEV, sft_rows=R)
    kw = {}
    if with_cache:
        kw = dict(cache_k=H.nan_like((B, Hkv, T, d), tdt, DEV),
                  cache_v=H.nan_like((B, Hkv, T, d), tdt, DEV),
                  cache_len=torch.zeros(B, dtype=torch.int32, device=DEV))
    out_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    ox.forward_sft(shape, q_base, q_out, out_pos, k, v, H.device_affine(inp["affine"], DEV),
                   ob, oo, ws, **kw)
    torch.cuda.synchronize()
    rb, ro = oracle.forward_sft(H.to64(inp["q_base"]), H.to64(inp["q_out"]), H.to64(inp["k"]),
                                H.to64(inp["v"]), pos, *H.affine64(inp["affine"]), window=w)
    H.assert_close(H.to64(ob), rb, tdt, "o_base")
    H.assert_close(H.to64(oo), ro, tdt, "o_out")
    if with_cache:
        np.testing.assert_array_equal(H.cache_as_tokens(kw["cache_k"], T), H.to64(inp["k"]))
        assert kw["cache_len"].cpu().tolist() == [T] * B


CHUNK_CASES = [
    # (B, Hq, Hkv, d, chunks, w, dtype)
    (2, 8, 2, 128, [100, 37, 200], 64, "bf16"),   # windows reach back across chunks
    (1, 4, 1, 128, [1, 1, 1, 70, 1], 16, "bf16"),  # single-token chunks
    (1, 4, 4, 128, [130, 130], 300, "bf16"),       # window longer than everything: causal
    (1, 4, 2, 64, [65, 64, 63], 65, "bf16"),       # d 64, tile-boundary chunk sizes
    (2, 4, 2, 64, [40, 33], 20, "f32"),            # fp32 rows
]


# last_only: the chunks before the last pass no output row (q_out = o_out = None), as a
# prompt's intermediate chunks need none; their base rows and the cache are still checked.
@pytest.mark.parametrize("B,Hq,Hkv,d,chunks,w,dt,last_only",
                         [c + (False,) for c in CHUNK_CASES] +
                         [CHUNK_CASES[0] + (True,), CHUNK_CASES[4] + (True,)])
def test_prefill_in_chunks_matches_oracle(B, Hq, Hkv, d, chunks, w, dt, last_only):
    P = sum(chunks)
    wl = _wl(mode="prefill", batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=d, length=P, window=w,
             dtype=dt, seed=600 + P)
    _say("prefill chunks", wl, chunks, "last only" if last_only else "")
    inp = syn.make_prefill(wl)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    cap = P + 3
    shape = ox.Shape(B, Hq, Hkv, d, w, tdt, cap)
    ck = H.nan_like((B, Hkv, cap, d), tdt, DEV)
    cv = H.nan_like((B, Hkv, cap, d), tdt, DEV)
    cl = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = ox.make_workspace(shape, DEV)
    aff = H.device_affine(inp["affine"], DEV)
    a64 = H.affine64(inp["affine"])
    g = torch.Generator().manual_seed(wl.seed + 1)
    hk = np.zeros((B, 0, Hkv, d))
    hv = np.zeros((B, 0, Hkv, d))
    past = 0
    for c in chunks:
        sl = slice(past, past + c)
        qo = torch.randn(B, 1, Hq, d, generator=g).to(tdt)
        ob = H.nan_like((B, c, Hq, d), tdt, DEV)
        oo = H.nan_like((B, 1, Hq, d), tdt, DEV)
        row = not last_only or past + c == P  # this chunk computes the output row
        ox.prefill_chunk(shape, past, inp["q_base"][:, sl].contiguous().to(DEV),
                         qo.to(DEV) if row else None,
                         inp["k"][:, sl].contiguous().to(DEV), inp["v"][:, sl].contiguous().to(DEV),
                         aff, ck, cv, cl, ob, oo if row else None, ws)
        torch.cuda.synchronize()
        rb, ro, hk, hv, rl = oracle.prefill_chunk(
            hk, hv, past, H.to64(inp["q_base"][:, sl]), H.to64(qo), H.to64(inp["k"][:, sl]),
            H.to64(inp["v"][:, sl]), *a64, window=w)
        H.assert_close(H.to64(ob), rb, tdt, f"o_base chunk at {past}")
        if row:
            H.assert_close(H.to64(oo), ro, tdt, f"o_out chunk at {past}")
        past += c
        assert cl.cpu().tolist() == rl.tolist()
    np.testing.assert_array_equal(H.cache_as_tokens(ck, P), hk)
    np.testing.assert_array_equal(H.cache_as_tokens(cv, P), hv)
