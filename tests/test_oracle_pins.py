"""Pins for the float64 oracle, checked against things other than the oracle itself.

Sources of truth, all CPU-only:
  * a hand-derived worked example (tests/golden/worked_example.json) for the paper
    "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers", §3.1 Eq. 4/5
    and the query scale-offset definitions;
  * torch's scaled_dot_product_attention in float64 (a library attention routine) with its own
    causal flag, its own grouped-query expansion, and an explicit band mask;
  * closed forms (zero keys give plain averages over the window or the prefix; window 1
    returns the value row);
  * invariants of the equations: window >= T is causal attention, GQA equals MHA with
    repeated key/value heads, linearity in V, weights form a distribution, the PT regime agrees
    with prefill followed by decode steps (§3.2), the SFT rows agree with PT rows, and a
    planted key matching the query dominates the output row.
Each pin is chosen so a plausible slip in the oracle (dropped offset, wrong scale, window off
by one, wrong head mapping, attend-before-append in decode, transposed operand) fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(1234)


def _val(x):
    if isinstance(x, str):
        return {"sqrt2": math.sqrt(2.0), "sqrt2-2": math.sqrt(2.0) - 2.0,
                "ln2": math.log(2.0), "ln3": math.log(3.0)}[x]
    return float(x)


def _arr(rows):
    return np.array([[_val(x) for x in r] for r in rows], dtype=np.float64)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _affine(hq, d, identity=False):
    if identity:
        return np.ones(hq * d), np.zeros(hq * d), np.ones(hq * d), np.zeros(hq * d)
    return (1 + 0.1 * _rand(hq * d), 0.1 * _rand(hq * d),
            1 + 0.1 * _rand(hq * d), 0.1 * _rand(hq * d))


# ---------------------------------------------------------------------------------------------
# Worked example (hand-derived, exact)
# ---------------------------------------------------------------------------------------------
def _golden():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        g = json.load(f)
    T = len(g["k"])
    qb = _arr(g["q_raw_base"]).reshape(1, T, 1, 2)
    qo = _arr(g["q_raw_out"]).reshape(1, T, 1, 2)
    k = _arr(g["k"]).reshape(1, T, 1, 2)
    v = _arr(g["v"]).reshape(1, T, 1, 2)
    aff = (np.array([_val(x) for x in g["alpha_base"]]), np.array([_val(x) for x in g["beta_base"]]),
           np.array([_val(x) for x in g["alpha_out"]]), np.array([_val(x) for x in g["beta_out"]]))
    return g, qb, qo, k, v, aff


def test_worked_example_pt():
    g, qb, qo, k, v, aff = _golden()
    ob, oo = oracle.forward_pt(qb, qo, k, v, *aff, window=g["window"])
    np.testing.assert_allclose(ob[0, :, 0], _arr(g["expected_base"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oo[0, :, 0], _arr(g["expected_out"]), rtol=0, atol=1e-12)


def test_worked_example_prefill():
    g, qb, qo, k, v, aff = _golden()
    ob, oo, ck, cv, ln = oracle.prefill(qb, qo[:, -1:], k, v, *aff, window=g["window"])
    np.testing.assert_allclose(ob[0, :, 0], _arr(g["expected_base"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oo[0, 0, 0], _arr(g["expected_out"])[-1], rtol=0, atol=1e-12)
    assert ln.tolist() == [3]
    np.testing.assert_array_equal(ck, k)
    np.testing.assert_array_equal(cv, v)


def test_worked_example_decode():
    """Prefill two tokens, decode the third: same rows as the hand derivation."""
    g, qb, qo, k, v, aff = _golden()
    _, _, ck, cv, ln = oracle.prefill(qb[:, :2], qo[:, 1:2], k[:, :2], v[:, :2], *aff,
                                      window=g["window"])
    ob, oo, nk, nv, nl = oracle.decode_step(ck, cv, ln, qb[:, 2], qo[:, 2], k[:, 2], v[:, 2],
                                            *aff, window=g["window"])
    np.testing.assert_allclose(ob[0, 0], _arr(g["expected_base"])[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(oo[0, 0], _arr(g["expected_out"])[2], rtol=0, atol=1e-12)
    assert nl.tolist() == [3]
    np.testing.assert_array_equal(nk[0], k[0])


# ---------------------------------------------------------------------------------------------
# Library routine: torch SDPA in float64
# ---------------------------------------------------------------------------------------------
def _sdpa(q, k, v, mask=None, causal=False, gqa=False):
    # q [T, Hq, d], k/v [T, Hkv, d] -> [T, Hq, d]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         is_causal=causal, enable_gqa=gqa)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("T,hq,hkv,d", [(37, 4, 1, 16), (50, 4, 2, 8), (64, 3, 3, 32)])
def test_output_stream_matches_sdpa_causal(T, hq, hkv, d):
    qb, qo = _rand(1, T, hq, d), _rand(1, T, hq, d)
    k, v = _rand(1, T, hkv, d), _rand(1, T, hkv, d)
    aff = _affine(hq, d)
    _, oo = oracle.forward_pt(qb, qo, k, v, *aff, window=5)
    q_eff = (aff[2].reshape(hq, d) * qo[0] + aff[3].reshape(hq, d))
    ref = _sdpa(q_eff, k[0], v[0], causal=True, gqa=hkv != hq)
    np.testing.assert_allclose(oo[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,w,hq,hkv,d", [(40, 1, 2, 1, 8), (40, 7, 4, 2, 16), (33, 32, 2, 2, 8),
                                          (33, 33, 2, 1, 8), (20, 64, 4, 4, 4)])
def test_base_stream_matches_sdpa_band(T, w, hq, hkv, d):
    qb, qo = _rand(1, T, hq, d), _rand(1, T, hq, d)
    k, v = _rand(1, T, hkv, d), _rand(1, T, hkv, d)
    aff = _affine(hq, d)
    ob, _ = oracle.forward_pt(qb, qo, k, v, *aff, window=w)
    q_eff = (aff[0].reshape(hq, d) * qb[0] + aff[1].reshape(hq, d))
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    band = (j <= t) & (j > t - w)
    ref = _sdpa(q_eff, k[0], v[0], mask=band, gqa=hkv != hq)
    np.testing.assert_allclose(ob[0], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,w", [(30, 1), (30, 4), (30, 29), (30, 30), (30, 100)])
def test_zero_keys_give_window_and_prefix_means(T, w):
    hq, hkv, d = 2, 1, 6
    qb, qo = _rand(1, T, hq, d), _rand(1, T, hq, d)
    k = np.zeros((1, T, hkv, d))
    v = _rand(1, T, hkv, d)
    ob, oo = oracle.forward_pt(qb, qo, k, v, *_affine(hq, d), window=w)
    c = np.concatenate([np.zeros((1, d)), np.cumsum(v[0, :, 0], axis=0)], axis=0)
    for t in range(T):
        lo = max(0, t - w + 1)
        np.testing.assert_allclose(ob[0, t, 0], (c[t + 1] - c[lo]) / (t + 1 - lo), atol=1e-12)
        np.testing.assert_allclose(ob[0, t, 1], (c[t + 1] - c[lo]) / (t + 1 - lo), atol=1e-12)
        np.testing.assert_allclose(oo[0, t, 1], c[t + 1] / (t + 1), atol=1e-12)


def test_window_one_returns_value_row():
    T, hq, hkv, d = 25, 4, 2, 8
    qb, qo, k, v = _rand(2, T, hq, d), _rand(2, T, hq, d), _rand(2, T, hkv, d), _rand(2, T, hkv, d)
    ob, _ = oracle.forward_pt(qb, qo, k, v, *_affine(hq, d), window=1)
    np.testing.assert_array_equal(ob, np.repeat(v, 2, axis=2))


def test_decode_zero_keys_mean_includes_new_token():
    """Eq. 4/5 upper limit j = t: the decode step's own key belongs to both windows."""
    B, L, hq, hkv, d, w = 2, 9, 2, 1, 4, 3
    ck, cv = np.zeros((B, L, hkv, d)), _rand(B, L, hkv, d)
    vn = _rand(B, hkv, d)
    ob, oo, _, nv, nl = oracle.decode_step(ck, cv, [L, L - 4], _rand(B, hq, d), _rand(B, hq, d),
                                           np.zeros((B, hkv, d)), vn, *_affine(hq, d), window=w)
    for b, Lb in enumerate([L, L - 4]):
        hist = np.concatenate([cv[b, :Lb, 0], vn[b, 0][None]], axis=0)
        np.testing.assert_allclose(ob[b, 0], hist[-w:].mean(0), atol=1e-12)
        np.testing.assert_allclose(oo[b, 1], hist.mean(0), atol=1e-12)
        assert nl[b] == Lb + 1 and len(nv[b]) == Lb + 1


# ---------------------------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------------------------
def test_window_at_least_T_is_causal_and_streams_coincide():
    T, hq, hkv, d = 31, 4, 2, 16
    q, k, v = _rand(1, T, hq, d), _rand(1, T, hkv, d), _rand(1, T, hkv, d)
    a, b = 1 + 0.1 * _rand(hq * d), 0.1 * _rand(hq * d)
    ob, oo = oracle.forward_pt(q, q, k, v, a, b, a, b, window=T)
    np.testing.assert_allclose(ob, oo, rtol=0, atol=1e-13)
    ob2, _ = oracle.forward_pt(q, q, k, v, a, b, a, b, window=10 * T)
    np.testing.assert_allclose(ob2, oo, rtol=0, atol=1e-13)


def test_identity_affine_is_plain_attention():
    """alpha = 1, beta = 0 is the paper's ablation without scale-offset (§4.1)."""
    T, hq, d = 12, 2, 8
    q, k, v = _rand(1, T, hq, d), _rand(1, T, hq, d), _rand(1, T, hq, d)
    _, oo = oracle.forward_pt(q, q, k, v, *_affine(hq, d, identity=True), window=3)
    np.testing.assert_allclose(oo[0], _sdpa(q[0], k[0], v[0], causal=True), atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    T, hq, hkv, d = 20, 8, 2, 8
    qb, qo, k, v = _rand(1, T, hq, d), _rand(1, T, hq, d), _rand(1, T, hkv, d), _rand(1, T, hkv, d)
    aff = _affine(hq, d)
    ob, oo = oracle.forward_pt(qb, qo, k, v, *aff, window=6)
    G = hq // hkv
    ob2, oo2 = oracle.forward_pt(qb, qo, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), *aff,
                                 window=6)
    np.testing.assert_array_equal(ob, ob2)
    np.testing.assert_array_equal(oo, oo2)


def test_linear_in_values():
    T, hq, d = 18, 2, 8
    qb, qo, k = _rand(1, T, hq, d), _rand(1, T, hq, d), _rand(1, T, hq, d)
    v1, v2 = _rand(1, T, hq, d), _rand(1, T, hq, d)
    aff = _affine(hq, d)
    r1 = oracle.forward_pt(qb, qo, k, v1, *aff, window=5)
    r2 = oracle.forward_pt(qb, qo, k, v2, *aff, window=5)
    r3 = oracle.forward_pt(qb, qo, k, 2.0 * v1 - 3.0 * v2, *aff, window=5)
    for a, b, c in zip(r1, r2, r3):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, atol=1e-12)


def test_weights_form_a_distribution():
    for n in (1, 2, 17, 300):
        w = oracle.attention_weights(_rand(16) * 3, _rand(n, 16) * 3, 0.25)
        assert np.all(w >= 0)
        assert abs(w.sum() - 1.0) < 1e-12


def test_pt_equals_prefill_then_decode():
    """§3.2: the four regimes are one formulation; batch PT rows equal incremental rows."""
    B, T, P0, hq, hkv, d, w = 2, 24, 9, 4, 2, 8, 5
    qb, qo, k, v = _rand(B, T, hq, d), _rand(B, T, hq, d), _rand(B, T, hkv, d), _rand(B, T, hkv, d)
    aff = _affine(hq, d)
    ob, oo = oracle.forward_pt(qb, qo, k, v, *aff, window=w)
    pb, po, ck, cv, ln = oracle.prefill(qb[:, :P0], qo[:, P0 - 1:P0], k[:, :P0], v[:, :P0], *aff,
                                        window=w)
    np.testing.assert_allclose(pb, ob[:, :P0], atol=1e-13)
    np.testing.assert_allclose(po[:, 0], oo[:, P0 - 1], atol=1e-13)
    hist_k, hist_v, lens = list(ck), list(cv), ln
    for t in range(P0, T):
        db, do, hist_k, hist_v, lens = oracle.decode_step(hist_k, hist_v, lens, qb[:, t], qo[:, t],
                                                          k[:, t], v[:, t], *aff, window=w)
        np.testing.assert_allclose(db, ob[:, t], atol=1e-13)
        np.testing.assert_allclose(do, oo[:, t], atol=1e-13)
    np.testing.assert_array_equal(np.stack(hist_k), k)


def test_sft_rows_equal_pt_rows():
    B, T, hq, hkv, d, w = 1, 20, 2, 1, 8, 4
    qb, qo, k, v = _rand(B, T, hq, d), _rand(B, T, hq, d), _rand(B, T, hkv, d), _rand(B, T, hkv, d)
    aff = _affine(hq, d)
    ob, oo = oracle.forward_pt(qb, qo, k, v, *aff, window=w)
    pos = [3, 11, 19]
    sb, so = oracle.forward_sft(qb, qo[:, pos], k, v, pos, *aff, window=w)
    np.testing.assert_allclose(sb, ob, atol=1e-13)
    np.testing.assert_allclose(so, oo[:, pos], atol=1e-13)


def test_planted_key_dominates_output_row():
    P, hq, hkv, d, w = 400, 4, 2, 128, 16
    qb, qo = _rand(1, P, hq, d), _rand(1, 1, hq, d)
    k, v = _rand(1, P, hkv, d), _rand(1, P, hkv, d)
    p = 37
    G = hq // hkv
    for g in range(hkv):
        k[0, p, g] = qo[0, 0, g * G]
    a, b = np.ones(hq * d), np.zeros(hq * d)
    _, oo, *_ = oracle.prefill(qb, qo, k, v, a, b, a, b, window=w)
    for g in range(hkv):
        wts = oracle.attention_weights(qo[0, 0, g * G], k[0, :, g], oracle.default_scale(d))
        assert int(np.argmax(wts)) == p
        assert wts[p] > 0.5
        np.testing.assert_allclose(oo[0, 0, g * G], wts @ v[0, :, g], atol=1e-12)


def test_sampled_rows_match_full_evaluation():
    """Row subsets (used for sampled checks at large sizes) equal the full evaluation."""
    B, T, hq, hkv, d, w = 1, 30, 2, 2, 8, 7
    qb, qo, k, v = _rand(B, T, hq, d), _rand(B, 1, hq, d), _rand(B, T, hkv, d), _rand(B, T, hkv, d)
    aff = _affine(hq, d)
    full = oracle.prefill(qb, qo, k, v, *aff, window=w)
    part = oracle.prefill(qb, qo, k, v, *aff, window=w, rows=[0, 6, 7, 29])
    for t in [0, 6, 7, 29]:
        np.testing.assert_array_equal(part[0][:, t], full[0][:, t])
    assert np.isnan(part[0][:, 1]).all()


@pytest.mark.parametrize("chunks,w", [([9, 7, 12], 5), ([1, 1, 30], 4), ([16, 16], 40), ([5], 3)])
def test_chunked_prefill_equals_one_shot_prefill(chunks, w):
    """§3.2 prefilling in pieces: each chunk's rows equal the one-shot prefill rows at the same
    positions, and the last chunk's output row equals the one-shot output row."""
    B, hq, hkv, d = 2, 4, 2, 8
    P = sum(chunks)
    qb, qo = _rand(B, P, hq, d), _rand(B, 1, hq, d)
    k, v = _rand(B, P, hkv, d), _rand(B, P, hkv, d)
    aff = _affine(hq, d)
    ob, oo, ck, cv, ln = oracle.prefill(qb, qo, k, v, *aff, window=w)
    hk, hv, past = np.zeros((B, 0, hkv, d)), np.zeros((B, 0, hkv, d)), 0
    for i, c in enumerate(chunks):
        sl = slice(past, past + c)
        q_o = qo if i == len(chunks) - 1 else _rand(B, 1, hq, d)
        cb, co, hk, hv, cl = oracle.prefill_chunk(hk, hv, past, qb[:, sl], q_o, k[:, sl], v[:, sl],
                                                  *aff, window=w)
        np.testing.assert_allclose(cb, ob[:, sl], atol=1e-13)
        past += c
        assert cl.tolist() == [past] * B
    np.testing.assert_allclose(co, oo, atol=1e-13)
    np.testing.assert_array_equal(hk, ck)
    np.testing.assert_array_equal(hv, cv)


def test_chunk_rows_match_sdpa_band_over_joined_sequence():
    """Library routine: a chunk after cached history is a band-masked SDPA over the joined keys,
    restricted to the chunk's query rows; its output row is the causal SDPA row at the end."""
    past, C, hq, hkv, d, w = 13, 10, 4, 1, 16, 6
    hk, hv = _rand(1, past, hkv, d), _rand(1, past, hkv, d)
    qb, qo = _rand(1, C, hq, d), _rand(1, 1, hq, d)
    k, v = _rand(1, C, hkv, d), _rand(1, C, hkv, d)
    aff = _affine(hq, d)
    cb, co, Kj, Vj, _ = oracle.prefill_chunk(hk, hv, past, qb, qo, k, v, *aff, window=w)
    n = past + C
    q_eff = aff[0].reshape(hq, d) * qb[0] + aff[1].reshape(hq, d)
    t = np.arange(past, n)[:, None]
    j = np.arange(n)[None, :]
    band = (j <= t) & (j > t - w)
    # SDPA with C query rows against n keys: pad the queries to n rows, take the chunk's rows
    qpad = np.zeros((n, hq, d))
    qpad[past:] = q_eff
    mpad = np.ones((n, n), dtype=bool)
    mpad[past:] = band
    ref = _sdpa(qpad, np.concatenate([hk[0], k[0]]), np.concatenate([hv[0], v[0]]), mask=mpad,
                gqa=True)[past:]
    np.testing.assert_allclose(cb[0], ref, rtol=0, atol=1e-12)
    qo_eff = aff[2].reshape(hq, d) * qo[0, 0] + aff[3].reshape(hq, d)
    ref_o = _sdpa(qo_eff[None], np.concatenate([hk[0], k[0]]), np.concatenate([hv[0], v[0]]),
                  gqa=True)[0]  # one query row sees every key 0 .. n-1
    np.testing.assert_allclose(co[0, 0], ref_o, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(Kj[0], np.concatenate([hk[0], k[0]]))


def _scatter_blocks(hist, table, pool_pages, ps):
    """Test-side construction of a paged pool: block i of the history (tokens i ps .. i ps +
    ps - 1, as a [H_kv, ps, d] slab) is copied whole into page table[i]. Written per block with
    slicing, independently of the oracle's per-token gather."""
    pool = np.asarray(pool_pages).copy()
    L = hist.shape[0]
    for i in range((L + ps - 1) // ps):
        blk = hist[i * ps:(i + 1) * ps]            # [n, H_kv, d]
        pool[table[i], :, :blk.shape[0], :] = np.transpose(blk, (1, 0, 2))
    return pool


@pytest.mark.parametrize("ps,lengths", [(1, [5, 9]), (4, [13, 8, 1]), (16, [40, 0]),
                                        (64, [30, 64])])
def test_gather_pages_inverts_a_block_scatter(ps, lengths):
    Hkv, d = 2, 8
    max_pages = max((L + ps - 1) // ps for L in lengths) + 1
    num_pages = len(lengths) * max_pages + 3
    perm = RNG.permutation(num_pages)
    table = perm[:len(lengths) * max_pages].reshape(len(lengths), max_pages)
    pool = RNG.standard_normal((num_pages, Hkv, ps, d))
    for b, L in enumerate(lengths):
        hist = RNG.standard_normal((L, Hkv, d))
        pooled = _scatter_blocks(hist, table[b], pool, ps)
        np.testing.assert_array_equal(oracle.gather_pages(pooled, table[b], L), hist)
        # pages outside this sequence's blocks are untouched by the scatter
        used = set(table[b][:(L + ps - 1) // ps].tolist())
        for pg in range(num_pages):
            if pg not in used:
                np.testing.assert_array_equal(pooled[pg], pool[pg])


@pytest.mark.parametrize("ps", [1, 8, 32])
def test_paged_decode_equals_contiguous_decode(ps):
    """Same outputs as decode_step over the gathered histories; the new token lands in exactly
    one slot per sequence (read back through the table); a full sequence writes nothing."""
    B, Hq, Hkv, d, w = 3, 4, 2, 8, 5
    max_pages = 40 // ps + 2
    cap = max_pages * ps
    lengths = [7, 33, cap]  # the last sequence is full
    num_pages = B * max_pages + 2
    table = RNG.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    kp = RNG.standard_normal((num_pages, Hkv, ps, d))
    vp = RNG.standard_normal((num_pages, Hkv, ps, d))
    hk = [RNG.standard_normal((L, Hkv, d)) for L in lengths]
    hv = [RNG.standard_normal((L, Hkv, d)) for L in lengths]
    for b in range(B):
        kp = _scatter_blocks(hk[b], table[b], kp, ps)
        vp = _scatter_blocks(hv[b], table[b], vp, ps)
    qb = RNG.standard_normal((B, Hq, d))
    qo = RNG.standard_normal((B, Hq, d))
    kn = RNG.standard_normal((B, Hkv, d))
    vn = RNG.standard_normal((B, Hkv, d))
    aff = [1 + 0.1 * RNG.standard_normal(Hq * d), 0.1 * RNG.standard_normal(Hq * d),
           1 + 0.1 * RNG.standard_normal(Hq * d), 0.1 * RNG.standard_normal(Hq * d)]
    ob, oo, kp2, vp2, lens, full = oracle.decode_step_paged(kp, vp, table, np.array(lengths),
                                                            qb, qo, kn, vn, *aff, window=w)
    rb, ro, _, _, _ = oracle.decode_step(hk, hv, np.array(lengths), qb, qo, kn, vn, *aff,
                                         window=w)
    np.testing.assert_array_equal(ob, rb)
    np.testing.assert_array_equal(oo, ro)
    assert lens.tolist() == [lengths[0] + 1, lengths[1] + 1, lengths[2]]
    assert full.tolist() == [False, False, True]
    for b in range(2):
        L = lengths[b]
        np.testing.assert_array_equal(oracle.gather_pages(kp2, table[b], L + 1),
                                      np.concatenate([hk[b], kn[b][None]]))
        np.testing.assert_array_equal(oracle.gather_pages(vp2, table[b], L + 1),
                                      np.concatenate([hv[b], vn[b][None]]))
    changed = np.argwhere(kp2 != kp)
    assert len({(int(c[0]), int(c[2])) for c in changed}) == 2  # one (page, slot) per written seq
    np.testing.assert_array_equal(kp2[table[2]], kp[table[2]])


# ---- training: backward pass and per-row log-sum-exp ----------------------------------------
def _train_case(B=1, T=8, Hq=2, Hkv=1, d=4, seed=5):
    r = np.random.default_rng(seed)
    x = dict(q_base=r.standard_normal((B, T, Hq, d)), q_out=r.standard_normal((B, T, Hq, d)),
             k=r.standard_normal((B, T, Hkv, d)), v=r.standard_normal((B, T, Hkv, d)),
             alpha_b=1 + 0.3 * r.standard_normal(Hq * d), beta_b=0.3 * r.standard_normal(Hq * d),
             alpha_o=1 + 0.3 * r.standard_normal(Hq * d), beta_o=0.3 * r.standard_normal(Hq * d))
    g = dict(do_base=r.standard_normal((B, T, Hq, d)), do_out=r.standard_normal((B, T, Hq, d)))
    return x, g


def _loss(x, g, w):
    ob, oo = oracle.forward_pt(x["q_base"], x["q_out"], x["k"], x["v"], x["alpha_b"],
                               x["beta_b"], x["alpha_o"], x["beta_o"], window=w)
    return float(np.sum(ob * g["do_base"]) + np.sum(oo * g["do_out"]))


_GRAD_OF = dict(q_base="dq_base", q_out="dq_out", k="dk", v="dv", alpha_b="dalpha_b",
                beta_b="dbeta_b", alpha_o="dalpha_o", beta_o="dbeta_o")


@pytest.mark.parametrize("w,Hq,Hkv,B", [(3, 2, 1, 1), (1, 2, 2, 1), (20, 4, 2, 2)])
def test_backward_matches_central_differences_of_the_forward(w, Hq, Hkv, B):
    """Every gradient entry equals the central difference of L = <do_base, o_base> +
    <do_out, o_out> computed with the (separately pinned) forward oracle."""
    x, g = _train_case(B=B, Hq=Hq, Hkv=Hkv, seed=10 + w)
    grads = oracle.backward_pt(x["q_base"], x["q_out"], x["k"], x["v"], x["alpha_b"],
                               x["beta_b"], x["alpha_o"], x["beta_o"], g["do_base"], g["do_out"],
                               window=w)
    h = 1e-5
    for name, gname in _GRAD_OF.items():
        arr = x[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(x, g, w)
            arr[idx] = keep - h
            lm = _loss(x, g, w)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[gname], num, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_backward_matches_torch_autograd_through_sdpa():
    """Gradients equal torch autograd (float64) through scaled_dot_product_attention with an
    explicit band mask (base stream) and its causal flag (output stream), GQA by repeating
    the kv heads."""
    B, T, Hq, Hkv, d, w = 2, 37, 4, 2, 8, 9
    x, g = _train_case(B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, seed=3)
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    G = Hq // Hkv
    K = t["k"].transpose(1, 2).repeat_interleave(G, dim=1)
    V = t["v"].transpose(1, 2).repeat_interleave(G, dim=1)
    qb = (t["alpha_b"].view(Hq, d) * t["q_base"] + t["beta_b"].view(Hq, d)).transpose(1, 2)
    qo = (t["alpha_o"].view(Hq, d) * t["q_out"] + t["beta_o"].view(Hq, d)).transpose(1, 2)
    i = torch.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - w)
    F = torch.nn.functional
    ob = F.scaled_dot_product_attention(qb, K, V, attn_mask=band)
    oo = F.scaled_dot_product_attention(qo, K, V, is_causal=True)
    loss = (ob * torch.tensor(g["do_base"]).transpose(1, 2)).sum() + \
           (oo * torch.tensor(g["do_out"]).transpose(1, 2)).sum()
    loss.backward()
    grads = oracle.backward_pt(x["q_base"], x["q_out"], x["k"], x["v"], x["alpha_b"],
                               x["beta_b"], x["alpha_o"], x["beta_o"], g["do_base"], g["do_out"],
                               window=w)
    for name, gname in _GRAD_OF.items():
        np.testing.assert_allclose(grads[gname], t[name].grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=gname)


def test_lse_matches_library_logsumexp():
    B, T, Hq, Hkv, d, w = 1, 30, 4, 2, 8, 7
    x, _ = _train_case(B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, seed=4)
    lb, lo = oracle.lse_pt(x["q_base"], x["q_out"], x["k"], x["alpha_b"], x["beta_b"],
                           x["alpha_o"], x["beta_o"], window=w)
    s = 1 / math.sqrt(d)
    i = torch.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - w)
    causal = i[None, :] <= i[:, None]
    for q_raw, a, bt, mask, got in ((x["q_base"], x["alpha_b"], x["beta_b"], band, lb),
                                    (x["q_out"], x["alpha_o"], x["beta_o"], causal, lo)):
        q = torch.tensor(a.reshape(Hq, d) * q_raw + bt.reshape(Hq, d))[0]  # [T, Hq, d]
        for h in range(Hq):
            kk = torch.tensor(x["k"][0, :, h // (Hq // Hkv)])
            z = s * q[:, h] @ kk.T
            z = z.masked_fill(~mask, float("-inf"))
            np.testing.assert_allclose(got[0, h], torch.logsumexp(z, dim=1).numpy(), rtol=1e-12)
    # a row with one key (t = 0) has lse equal to its only score
    q0 = x["alpha_b"].reshape(Hq, d) * x["q_base"][0, 0] + x["beta_b"].reshape(Hq, d)
    np.testing.assert_allclose(lb[0, 0, 0], s * q0[0] @ x["k"][0, 0, 0], rtol=1e-12)


def _sft_loss(x, g, pos, w):
    ob, oo = oracle.forward_sft(x["q_base"], x["q_out"], x["k"], x["v"], pos, x["alpha_b"],
                                x["beta_b"], x["alpha_o"], x["beta_o"], window=w)
    return float(np.sum(ob * g["do_base"]) + np.sum(oo * g["do_out"]))


@pytest.mark.parametrize("pos,w", [([7, 2, 5], 3), ([0], 2), ([4, 4, 7, 1], 8)])
def test_sft_backward_matches_central_differences(pos, w):
    """SFT gradients (response rows in any order, repeats allowed) against central differences
    of the separately pinned SFT forward."""
    x, g = _train_case(B=1, T=8, Hq=2, Hkv=1, d=4, seed=30 + w)
    r = np.random.default_rng(31)
    R = len(pos)
    x["q_out"] = r.standard_normal((1, R, 2, 4))
    g["do_out"] = r.standard_normal((1, R, 2, 4))
    grads = oracle.backward_sft(x["q_base"], x["q_out"], x["k"], x["v"], pos, x["alpha_b"],
                                x["beta_b"], x["alpha_o"], x["beta_o"], g["do_base"],
                                g["do_out"], window=w)
    h = 1e-5
    for name, gname in _GRAD_OF.items():
        arr = x[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _sft_loss(x, g, pos, w)
            arr[idx] = keep - h
            lm = _sft_loss(x, g, pos, w)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[gname], num, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_sft_backward_with_every_position_is_pt_backward():
    x, g = _train_case(B=2, T=12, Hq=4, Hkv=2, d=4, seed=8)
    T = 12
    a = oracle.backward_sft(x["q_base"], x["q_out"], x["k"], x["v"], list(range(T)), x["alpha_b"],
                            x["beta_b"], x["alpha_o"], x["beta_o"], g["do_base"], g["do_out"],
                            window=5)
    b = oracle.backward_pt(x["q_base"], x["q_out"], x["k"], x["v"], x["alpha_b"], x["beta_b"],
                           x["alpha_o"], x["beta_o"], g["do_base"], g["do_out"], window=5)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    la = oracle.lse_sft(x["q_base"], x["q_out"], x["k"], list(range(T)), x["alpha_b"],
                        x["beta_b"], x["alpha_o"], x["beta_o"], window=5)
    lb = oracle.lse_pt(x["q_base"], x["q_out"], x["k"], x["alpha_b"], x["beta_b"], x["alpha_o"],
                       x["beta_o"], window=5)
    np.testing.assert_array_equal(la[1], lb[1])
    np.testing.assert_array_equal(la[0], lb[0])


def test_lse_sft_rows_match_library_logsumexp():
    """Output rows at unsorted and repeated response positions (Eq. 5 ranges, keys 0 .. pos)
    and every base row (Eq. 4 ranges) against torch.logsumexp over explicitly masked scores."""
    B, T, Hq, Hkv, d, w = 2, 14, 4, 2, 8, 4
    x, _ = _train_case(B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, seed=12)
    pos = [9, 0, 13, 9, 3, 13, 6]
    R = len(pos)
    r = np.random.default_rng(13)
    x["q_out"] = r.standard_normal((B, R, Hq, d))
    lb, lo = oracle.lse_sft(x["q_base"], x["q_out"], x["k"], pos, x["alpha_b"], x["beta_b"],
                            x["alpha_o"], x["beta_o"], window=w)
    assert lb.shape == (B, Hq, T) and lo.shape == (B, Hq, R)
    s = 1 / math.sqrt(d)
    i = torch.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - w)
    rows = torch.tensor(pos)
    prefix = i[None, :] <= rows[:, None]  # [R, T]
    for b in range(B):
        qb = torch.tensor(x["alpha_b"].reshape(Hq, d) * x["q_base"][b] + x["beta_b"].reshape(Hq, d))
        qo = torch.tensor(x["alpha_o"].reshape(Hq, d) * x["q_out"][b] + x["beta_o"].reshape(Hq, d))
        for h in range(Hq):
            kk = torch.tensor(x["k"][b, :, h // (Hq // Hkv)])
            zb = (s * qb[:, h] @ kk.T).masked_fill(~band, float("-inf"))
            np.testing.assert_allclose(lb[b, h], torch.logsumexp(zb, dim=1).numpy(), rtol=1e-12)
            zo = (s * qo[:, h] @ kk.T).masked_fill(~prefix, float("-inf"))
            np.testing.assert_allclose(lo[b, h], torch.logsumexp(zo, dim=1).numpy(), rtol=1e-12)
    # repeated positions with the same query give the same value; row 1 (position 0) is its score
    np.testing.assert_allclose(lo[:, :, 1],
                               s * np.einsum("bhd,bhd->bh",
                                             x["alpha_o"].reshape(Hq, d) * x["q_out"][:, 1]
                                             + x["beta_o"].reshape(Hq, d),
                                             np.repeat(x["k"][:, 0], Hq // Hkv, axis=1)),
                               rtol=1e-12)


@pytest.mark.parametrize("ps,T", [(1, 3), (4, 6), (8, 5), (16, 17)])
def test_paged_write_appends_tokens_across_pages(ps, T):
    """A T-token append per sequence, read back through the table, equals history + tokens
    (a write that crosses page boundaries included); a sequence without room for all T tokens
    is left untouched and flagged; no page outside a sequence's written blocks changes."""
    B, Hkv, d = 4, 2, 4
    max_pages = 24 // ps + 2
    cap = max_pages * ps
    lengths = [ps - 1, 0, cap - T + 1, cap - T]  # crosses a page; empty; one short; exact fit
    num_pages = B * max_pages + 3
    table = RNG.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    kp = RNG.standard_normal((num_pages, Hkv, ps, d))
    vp = RNG.standard_normal((num_pages, Hkv, ps, d))
    hk = [RNG.standard_normal((L, Hkv, d)) for L in lengths]
    hv = [RNG.standard_normal((L, Hkv, d)) for L in lengths]
    for b in range(B):
        kp = _scatter_blocks(hk[b], table[b], kp, ps)
        vp = _scatter_blocks(hv[b], table[b], vp, ps)
    k = RNG.standard_normal((B, T, Hkv, d))
    v = RNG.standard_normal((B, T, Hkv, d))
    kp2, vp2, lens, full = oracle.paged_write(kp, vp, table, np.array(lengths), k, v)
    assert full.tolist() == [False, False, True, False]
    assert lens.tolist() == [lengths[0] + T, T, lengths[2], cap]
    for b in (0, 1, 3):
        L = lengths[b]
        # the expected pool: the whole new history scattered block by block by the test
        exp_k = _scatter_blocks(np.concatenate([hk[b], k[b]]), table[b], kp, ps)
        exp_v = _scatter_blocks(np.concatenate([hv[b], v[b]]), table[b], vp, ps)
        blocks = table[b][:(L + T + ps - 1) // ps]
        np.testing.assert_array_equal(kp2[blocks], exp_k[blocks])
        np.testing.assert_array_equal(vp2[blocks], exp_v[blocks])
        np.testing.assert_array_equal(oracle.gather_pages(kp2, table[b], L + T),
                                      np.concatenate([hk[b], k[b]]))
        np.testing.assert_array_equal(oracle.gather_pages(vp2, table[b], L + T),
                                      np.concatenate([hv[b], v[b]]))
    written = set()
    for b in (0, 1, 3):
        L = lengths[b]
        written |= {int(table[b][t // ps]) for t in range(L, L + T)}
    for pg in range(num_pages):
        if pg not in written:
            np.testing.assert_array_equal(kp2[pg], kp[pg])
            np.testing.assert_array_equal(vp2[pg], vp[pg])
    # the slots written are exactly positions L .. L + T - 1 of the written sequences
    changed = {(int(c[0]), int(c[1])) for c in np.argwhere((kp2 != kp).any(axis=(1, 3)))}
    expect = {(int(table[b][t // ps]), t % ps) for b in (0, 1, 3)
              for t in range(lengths[b], lengths[b] + T)}
    assert changed == expect
