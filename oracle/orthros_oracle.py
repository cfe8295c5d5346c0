"""Float64 CPU oracle for Orthros attention — TEST INFRASTRUCTURE, not product code.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import
this module. The product path (the HIP library and its Python binding) never calls it, and it
imports nothing from the product path.

What it computes follows the paper "Orthros: Phase-Aware Heterogeneous Attention for
Efficient Transformers":
  * §3.1, the query definitions: base query q_i = alpha (.) (x_i W_Q) + beta, output-stream
    query q'_i = alpha' (.) (x'_i W_Q) + beta'. Here the projection x W_Q is the caller's
    input ``q_raw``; the oracle applies only the element-wise scale-offset.
  * §3.1 Eq. 4: base-stream sliding-window attention; row t sees keys
    max(1, t-w+1) .. t (1-based), i.e. exactly w keys including itself.
  * §3.1 Eq. 5: output-stream full causal cross-attention; row t sees keys 1 .. t.
  * §3.1: keys and values come from the base tokens only; the output stream never writes
    them (Algorithm 1, the "shared KV cache" step).
  * §3.2: the regimes Pre-Training (every position duplicated), Prefilling (one output row
    at the last prompt token) and Decoding (one new token, duplicated into a base copy that
    updates the cache and runs the window, and an output copy that attends to the history).
  * §3.2 SFT regime: output rows only at the response positions.
  * §3.2 Prefilling with the prompt arriving in chunks: the chunk's base tokens append their
    keys/values after the cached ones and run their windows over history plus chunk; one
    output row at the chunk's last token sees every key.
  * §3.2 Pre-Training is a training regime (the loss is taken at every position) and §3.1
    makes alpha, beta, alpha', beta' learnable: the backward pass gives the gradients of both
    streams with respect to the raw queries, the shared keys and values and the four
    scale-offset vectors, and the training forward the per-row log-sum-exp it reuses.
  * §3.2 Decoding over a paged cache (the batched serving setting §5 names as future work):
    the same decode step, with each sequence's history stored in fixed-size pages of a shared
    pool and found through a per-sequence table of page indices.

Readings where the pages are silent or garbled (all listed in the repository's design notes):
  * scale: the extracted equations lost the square root and the division; the scale is the
    usual 1/sqrt(d_h) unless the caller passes another one.
  * positions are 0-based here: row t (0-based) of Eq. 4 sees keys max(0, t-w+1) .. t.
  * grouped-query attention (absent from the pages): query head h reads key/value head
    h // (H_q / H_kv).
  * the scale-offset vectors hold one entry per (query head, channel): shape [H_q * d].
  * "historical cache" in the decoding regime includes the current token (Eq. 5's upper
    limit j = t), so a decode step appends the new key/value before attending.

All arithmetic is float64 numpy. Inputs are converted to float64 exactly (bf16 and fp32
values are representable). No blocking, fusion or reordering beyond a per-row evaluation.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "default_scale",
    "scale_offset",
    "attention_weights",
    "attend",
    "base_row",
    "output_row",
    "prefill",
    "decode_step",
    "forward_pt",
    "forward_sft",
    "prefill_chunk",
    "gather_pages",
    "paged_write",
    "decode_step_paged",
    "lse_pt",
    "backward_pt",
    "lse_sft",
    "backward_sft",
]


def default_scale(head_dim: int) -> float:
    """Score scale 1/sqrt(d_h) (§3.1 Eq. 4/5; the root was lost in extraction)."""
    return 1.0 / np.sqrt(float(head_dim))


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scale_offset(q_raw, alpha, beta) -> np.ndarray:
    """§3.1: q = alpha (.) q_raw + beta, element-wise per (query head, channel).

    q_raw: [..., H_q, d]; alpha, beta: [H_q * d] (one entry per head and channel).
    """
    q_raw = _f64(q_raw)
    hq, d = q_raw.shape[-2], q_raw.shape[-1]
    a = _f64(alpha).reshape(hq, d)
    b = _f64(beta).reshape(hq, d)
    return a * q_raw + b


def attention_weights(q, K, scale) -> np.ndarray:
    """Softmax weights of Eq. 4/5 for one query vector q [d] over key rows K [n, d].

    exp(s q.k_j) / sum_m exp(s q.k_m). Every exponent is shifted by the same constant (the
    largest score) before exponentiation; the shift cancels between numerator and
    denominator and only keeps exp() finite.
    """
    z = scale * (_f64(K) @ _f64(q))
    e = np.exp(z - z.max())
    return e / e.sum()


def attend(q, K, V, scale) -> np.ndarray:
    """Eq. 4/5 for one query vector: sum_j softmax_j * v_j over the given rows."""
    w = attention_weights(q, K, scale)
    return w @ _f64(V)


def _kv_head(h: int, hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    return h // (hq // hkv)


def base_row(q_t, K, V, t: int, window: int, scale) -> np.ndarray:
    """Eq. 4 at 0-based position t for all query heads.

    q_t: [H_q, d] (already scale-offset); K, V: [n, H_kv, d] holding keys 0..t at least.
    Keys max(0, t-w+1) .. t.
    """
    lo = max(0, t - window + 1)
    return _rows_over(q_t, K[lo:t + 1], V[lo:t + 1], scale)


def output_row(q_t, K, V, t: int, scale) -> np.ndarray:
    """Eq. 5 at 0-based position t for all query heads: keys 0 .. t."""
    return _rows_over(q_t, K[:t + 1], V[:t + 1], scale)


def _rows_over(q_t, Kw, Vw, scale) -> np.ndarray:
    q_t = _f64(q_t)
    hq, d = q_t.shape
    hkv = Kw.shape[1]
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        out[h] = attend(q_t[h], Kw[:, g, :], Vw[:, g, :], scale)
    return out


def prefill(q_base, q_out, k, v, alpha_b, beta_b, alpha_o, beta_o, window, scale=None,
            rows=None):
    """§3.2 Prefilling (T_in = P-1, T_out = 1) for a batch of prompts of length P.

    q_base: [B, P, H_q, d] base-stream raw queries; q_out: [B, 1, H_q, d] raw query of the
    duplicated last prompt token; k, v: [B, P, H_kv, d].
    Returns (o_base [B, P, H_q, d], o_out [B, 1, H_q, d], cache_k, cache_v, cache_len) where
    the cache holds every prompt key/value (the base tokens write it; the output copy does
    not) and cache_len[b] = P.
    ``rows``: optional iterable of base positions to evaluate (others left NaN), for
    sampled checks at large P.
    """
    k = _f64(k)
    v = _f64(v)
    B, P = k.shape[0], k.shape[1]
    d = k.shape[-1]
    s = default_scale(d) if scale is None else scale
    qb = scale_offset(q_base, alpha_b, beta_b) if rows is None else None
    o_base = np.full(np.shape(q_base), np.nan)
    o_out = np.empty(np.shape(q_out))
    positions = range(P) if rows is None else rows
    for b in range(B):
        for t in positions:
            q_t = qb[b, t] if qb is not None else scale_offset(q_base[b, t], alpha_b, beta_b)
            o_base[b, t] = base_row(q_t, k[b], v[b], t, window, s)
        q_o = scale_offset(q_out[b, 0], alpha_o, beta_o)
        o_out[b, 0] = output_row(q_o, k[b], v[b], P - 1, s)
    cache_len = np.full(B, P, dtype=np.int64)
    return o_base, o_out, k.copy(), v.copy(), cache_len


def decode_step(cache_k, cache_v, cache_len, q_base, q_out, k_new, v_new,
                alpha_b, beta_b, alpha_o, beta_o, window, scale=None):
    """§3.2 Decoding (T = 1): one new token per sequence, duplicated into a pair.

    cache_k, cache_v: [B, >=L_b, H_kv, d] history; cache_len: [B] current lengths L_b.
    q_base, q_out: [B, H_q, d]; k_new, v_new: [B, H_kv, d].
    The base copy appends (k_new, v_new) at index L_b (its own key belongs to its window, the
    upper limit j = t of Eq. 4), then attends over max(0, L_b-w+1) .. L_b (Eq. 4); the output
    copy attends over 0 .. L_b (Eq. 5) and writes nothing.
    Returns (o_base [B, H_q, d], o_out [B, H_q, d], new_k_list, new_v_list, new_len) with the
    appended histories as a list of [L_b+1, H_kv, d] arrays.
    """
    B = len(cache_len)
    d = np.shape(q_base)[-1]
    s = default_scale(d) if scale is None else scale
    o_base = np.empty(np.shape(q_base))
    o_out = np.empty(np.shape(q_out))
    ks, vs, lens = [], [], []
    for b in range(B):
        L = int(cache_len[b])
        Kb = np.concatenate([_f64(cache_k[b][:L]), _f64(k_new[b])[None]], axis=0)
        Vb = np.concatenate([_f64(cache_v[b][:L]), _f64(v_new[b])[None]], axis=0)
        o_base[b] = base_row(scale_offset(q_base[b], alpha_b, beta_b), Kb, Vb, L, window, s)
        o_out[b] = output_row(scale_offset(q_out[b], alpha_o, beta_o), Kb, Vb, L, s)
        ks.append(Kb)
        vs.append(Vb)
        lens.append(L + 1)
    return o_base, o_out, ks, vs, np.asarray(lens, dtype=np.int64)


def forward_pt(q_base, q_out, k, v, alpha_b, beta_b, alpha_o, beta_o, window, scale=None,
               base_rows=None, out_rows=None):
    """§3.2 Pre-Training (T_in = 0, T_out = T): the whole sequence is duplicated.

    Base rows run Eq. 4 at every position with q_base; output rows run Eq. 5 at every position
    with q_out. Shapes: q_base, q_out [B, T, H_q, d]; k, v [B, T, H_kv, d].
    ``base_rows`` / ``out_rows``: optional position subsets (others left NaN).
    """
    k = _f64(k)
    v = _f64(v)
    B, T = k.shape[0], k.shape[1]
    d = k.shape[-1]
    s = default_scale(d) if scale is None else scale
    o_base = np.full(np.shape(q_base), np.nan)
    o_out = np.full(np.shape(q_out), np.nan)
    for b in range(B):
        for t in (range(T) if base_rows is None else base_rows):
            o_base[b, t] = base_row(scale_offset(q_base[b, t], alpha_b, beta_b), k[b], v[b],
                                    t, window, s)
        for t in (range(T) if out_rows is None else out_rows):
            o_out[b, t] = output_row(scale_offset(q_out[b, t], alpha_o, beta_o), k[b], v[b],
                                     t, s)
    return o_base, o_out


def forward_sft(q_base, q_out, k, v, out_positions, alpha_b, beta_b, alpha_o, beta_o,
                window, scale=None):
    """§3.2 Supervised Fine-Tuning (T_in = T - T_out, T_out >= 1).

    Base rows at every position (Eq. 4); output rows only at ``out_positions`` (Eq. 5), with
    q_out [B, T_out, H_q, d] holding the duplicated tokens in that order.
    """
    k = _f64(k)
    v = _f64(v)
    B, T = k.shape[0], k.shape[1]
    d = k.shape[-1]
    s = default_scale(d) if scale is None else scale
    o_base = np.empty(np.shape(q_base))
    o_out = np.empty(np.shape(q_out))
    for b in range(B):
        for t in range(T):
            o_base[b, t] = base_row(scale_offset(q_base[b, t], alpha_b, beta_b), k[b], v[b],
                                    t, window, s)
        for r, t in enumerate(out_positions):
            o_out[b, r] = output_row(scale_offset(q_out[b, r], alpha_o, beta_o), k[b], v[b],
                                     int(t), s)
    return o_base, o_out


def prefill_chunk(hist_k, hist_v, past_len, q_base, q_out, k, v, alpha_b, beta_b, alpha_o,
                  beta_o, window, scale=None):
    """§3.2 Prefilling for C more prompt tokens of sequences that already hold past_len.

    hist_k, hist_v: [B, >=past_len, H_kv, d] cached history (rows 0 .. past_len-1 are used);
    q_base [B, C, H_q, d]; q_out [B, 1, H_q, d] (the duplicated last token of the chunk);
    k, v [B, C, H_kv, d]. The chunk's keys/values follow the history at positions
    past_len .. past_len+C-1; base row i (position past_len + i) runs Eq. 4 over the joined
    sequence, and the output row runs Eq. 5 at position past_len + C - 1.
    Returns (o_base [B, C, H_q, d], o_out [B, 1, H_q, d], cache_k, cache_v, cache_len) with the
    joined [B, past_len + C, H_kv, d] history.
    """
    k = _f64(k)
    v = _f64(v)
    B, C = k.shape[0], k.shape[1]
    d = k.shape[-1]
    s = default_scale(d) if scale is None else scale
    Kj = np.concatenate([_f64(hist_k)[:, :past_len], k], axis=1)
    Vj = np.concatenate([_f64(hist_v)[:, :past_len], v], axis=1)
    o_base = np.empty(np.shape(q_base))
    o_out = np.empty(np.shape(q_out))
    for b in range(B):
        for i in range(C):
            o_base[b, i] = base_row(scale_offset(q_base[b, i], alpha_b, beta_b), Kj[b], Vj[b],
                                    past_len + i, window, s)
        o_out[b, 0] = output_row(scale_offset(q_out[b, 0], alpha_o, beta_o), Kj[b], Vj[b],
                                 past_len + C - 1, s)
    return o_base, o_out, Kj, Vj, np.full(B, past_len + C, dtype=np.int64)


def gather_pages(pages, table_row, length) -> np.ndarray:
    """History of one sequence read out of a paged cache, as [length, H_kv, d] float64.

    pages: [num_pages, H_kv, page_size, d] pool; table_row: page index of each logical block
    of the sequence. Token t sits in page table_row[t // page_size] at slot t % page_size.
    """
    pages = np.asarray(pages)
    ps = pages.shape[2]
    rows = []
    for t in range(int(length)):
        rows.append(_f64(pages[int(table_row[t // ps]), :, t % ps, :]))
    if not rows:
        return np.zeros((0, pages.shape[1], pages.shape[3]))
    return np.stack(rows)


def paged_write(k_pages, v_pages, table, cache_len, k, v):
    """Append T tokens per sequence to a paged cache (prefilling or decoding into pages).

    k_pages, v_pages [num_pages, H_kv, page_size, d]; table [B, max_pages]; cache_len [B];
    k, v [B, T, H_kv, d]. Tokens go to positions cache_len[b] .. cache_len[b] + T - 1. A
    sequence without room for all T tokens (capacity max_pages * page_size) is left unchanged
    and reported as full. Returns (new k_pages, new v_pages, new lengths, full flags) as
    float64 copies; the inputs are not modified.
    """
    kp = _f64(k_pages).copy()
    vp = _f64(v_pages).copy()
    k = _f64(k)
    v = _f64(v)
    B, T = k.shape[0], k.shape[1]
    ps = kp.shape[2]
    cap = np.shape(table)[1] * ps
    lens = np.asarray(cache_len, dtype=np.int64).copy()
    full = np.zeros(B, dtype=bool)
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L + T > cap:
            full[b] = True
            continue
        for i in range(T):
            t = L + i
            page = int(table[b][t // ps])
            kp[page, :, t % ps, :] = k[b, i]
            vp[page, :, t % ps, :] = v[b, i]
        lens[b] = L + T
    return kp, vp, lens, full


def decode_step_paged(k_pages, v_pages, table, cache_len, q_base, q_out, k_new, v_new,
                      alpha_b, beta_b, alpha_o, beta_o, window, scale=None):
    """§3.2 Decoding with the history in a paged cache.

    The attention outputs are those of ``decode_step`` over each sequence's gathered history
    (the new key L is this step's k_new, v_new); the new token is then written to position L
    through the table (nothing is written for a full sequence).
    Returns (o_base, o_out, new k_pages, new v_pages, new lengths, full flags).
    """
    B = len(cache_len)
    hk = [gather_pages(k_pages, table[b], cache_len[b]) for b in range(B)]
    hv = [gather_pages(v_pages, table[b], cache_len[b]) for b in range(B)]
    o_base, o_out, _, _, _ = decode_step(hk, hv, cache_len, q_base, q_out, k_new, v_new,
                                         alpha_b, beta_b, alpha_o, beta_o, window, scale)
    kp, vp, lens, full = paged_write(k_pages, v_pages, table, cache_len,
                                     _f64(k_new)[:, None], _f64(v_new)[:, None])
    return o_base, o_out, kp, vp, lens, full


def _stream_rows(T: int, window):
    """Key range [lo, t] of every row t: Eq. 4 with a window, Eq. 5 (window None) without."""
    return [(0 if window is None else max(0, t - window + 1), t) for t in range(T)]


def lse_pt(q_base, q_out, k, alpha_b, beta_b, alpha_o, beta_o, window, scale=None):
    """Per-row log-sum-exp (natural log) of the scaled scores s q_t . k_j over each row's keys,
    for the base rows (Eq. 4 ranges) and the output rows (Eq. 5 ranges) of the Pre-Training
    regime. Returns (lse_base, lse_out), each [B, H_q, T]."""
    k = _f64(k)
    B, T, hq, d = np.shape(q_base)
    hkv = k.shape[2]
    s = default_scale(d) if scale is None else scale
    out = []
    for q_raw, a, bt, w in ((q_base, alpha_b, beta_b, window), (q_out, alpha_o, beta_o, None)):
        q = scale_offset(q_raw, a, bt)
        lse = np.empty((B, hq, T))
        for b in range(B):
            for h in range(hq):
                g = _kv_head(h, hq, hkv)
                for t, (lo, hi) in enumerate(_stream_rows(T, w)):
                    z = s * (k[b, lo:hi + 1, g] @ q[b, t, h])
                    m = z.max()
                    lse[b, h, t] = m + np.log(np.exp(z - m).sum())
        out.append(lse)
    return out[0], out[1]


def _row_ranges(positions, window):
    """Key range [lo, t] of rows at the given positions (window None: Eq. 5, all keys <= t)."""
    return [(0 if window is None else max(0, int(t) - window + 1), int(t)) for t in positions]


def _stream_backward(q_raw, a, bt, K, V, dO, window, s, positions=None):
    """Backward of one stream for one (sequence, query head).

    q_raw [R, d] raw queries with their scale-offset a, bt [d] (R = T rows at positions
    0 .. T-1, or the rows at ``positions``); K, V [T, d] of the kv head; dO [R, d] the gradient
    of the loss with respect to the stream's outputs. With
    q = a (.) q_raw + bt, P the row-softmax weights of s q K^T over each row's keys and
    O = P V: dV = P^T dO; dP = dO V^T; the softmax Jacobian gives
    dZ_tj = P_tj (dP_tj - sum_m P_tm dP_tm); dq = s dZ K; dK = s dZ^T q; and through the
    scale-offset dq_raw = a (.) dq, da = sum_t dq (.) q_raw, db = sum_t dq.
    """
    q = a * q_raw + bt
    T = K.shape[0]
    ranges = _stream_rows(T, window) if positions is None else _row_ranges(positions, window)
    P = np.zeros((len(ranges), T))
    for r, (lo, hi) in enumerate(ranges):
        P[r, lo:hi + 1] = attention_weights(q[r], K[lo:hi + 1], s)
    dV = P.T @ dO
    dP = dO @ V.T
    dZ = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    dq = s * (dZ @ K)
    dK = s * (dZ.T @ q)
    return a * dq, np.sum(dq * q_raw, axis=0), np.sum(dq, axis=0), dK, dV


def backward_pt(q_base, q_out, k, v, alpha_b, beta_b, alpha_o, beta_o, do_base, do_out,
                window, scale=None):
    """Gradients of the Pre-Training regime's two streams (§3.2) for the output gradients
    do_base, do_out [B, T, H_q, d].

    Returns a dict with dq_base, dq_out [B, T, H_q, d] (with respect to the raw queries, before
    the scale-offset), dk, dv [B, T, H_kv, d] (both streams' contributions, summed over the
    query heads that share each kv head) and dalpha_b, dbeta_b, dalpha_o, dbeta_o [H_q * d]
    (summed over sequences and positions).
    """
    k = _f64(k)
    v = _f64(v)
    B, T, hq, d = np.shape(q_base)
    hkv = k.shape[2]
    s = default_scale(d) if scale is None else scale
    res = dict(dq_base=np.zeros((B, T, hq, d)), dq_out=np.zeros((B, T, hq, d)),
               dk=np.zeros((B, T, hkv, d)), dv=np.zeros((B, T, hkv, d)))
    for name, q_raw, a, bt, dO, w in (("b", q_base, alpha_b, beta_b, do_base, window),
                                      ("o", q_out, alpha_o, beta_o, do_out, None)):
        q_raw = _f64(q_raw)
        dO = _f64(dO)
        A = _f64(a).reshape(hq, d)
        Bt = _f64(bt).reshape(hq, d)
        da = np.zeros((hq, d))
        db = np.zeros((hq, d))
        dq_all = res["dq_base" if name == "b" else "dq_out"]
        for b in range(B):
            for h in range(hq):
                g = _kv_head(h, hq, hkv)
                dqr, dah, dbh, dK, dV = _stream_backward(q_raw[b, :, h], A[h], Bt[h], k[b, :, g],
                                                         v[b, :, g], dO[b, :, h], w, s)
                dq_all[b, :, h] = dqr
                da[h] += dah
                db[h] += dbh
                res["dk"][b, :, g] += dK
                res["dv"][b, :, g] += dV
        res["dalpha_" + name] = da.reshape(-1)
        res["dbeta_" + name] = db.reshape(-1)
    return res


def lse_sft(q_base, q_out, k, out_positions, alpha_b, beta_b, alpha_o, beta_o, window,
            scale=None):
    """Per-row log-sum-exp of the Supervised Fine-Tuning regime (§3.2): base rows at every
    position ([B, H_q, T], Eq. 4 ranges) and output rows at the response positions
    ([B, H_q, R], Eq. 5 ranges, in the order of ``out_positions``)."""
    k = _f64(k)
    B, T, hq, d = np.shape(q_base)
    hkv = k.shape[2]
    s = default_scale(d) if scale is None else scale
    out = []
    for q_raw, a, bt, ranges in ((q_base, alpha_b, beta_b, _stream_rows(T, window)),
                                 (q_out, alpha_o, beta_o, _row_ranges(out_positions, None))):
        q = scale_offset(q_raw, a, bt)
        lse = np.empty((B, hq, len(ranges)))
        for b in range(B):
            for h in range(hq):
                g = _kv_head(h, hq, hkv)
                for r, (lo, hi) in enumerate(ranges):
                    z = s * (k[b, lo:hi + 1, g] @ q[b, r, h])
                    m = z.max()
                    lse[b, h, r] = m + np.log(np.exp(z - m).sum())
        out.append(lse)
    return out[0], out[1]


def backward_sft(q_base, q_out, k, v, out_positions, alpha_b, beta_b, alpha_o, beta_o, do_base,
                 do_out, window, scale=None):
    """Gradients of the Supervised Fine-Tuning regime (§3.2): base rows at every position
    (Eq. 4), output rows only at ``out_positions`` (Eq. 5) with q_out, do_out [B, R, H_q, d].

    Same quantities as ``backward_pt`` (dq_out is [B, R, H_q, d]); with every position listed
    in order it is ``backward_pt``.
    """
    k = _f64(k)
    v = _f64(v)
    B, T, hq, d = np.shape(q_base)
    R = np.shape(q_out)[1]
    hkv = k.shape[2]
    s = default_scale(d) if scale is None else scale
    res = dict(dq_base=np.zeros((B, T, hq, d)), dq_out=np.zeros((B, R, hq, d)),
               dk=np.zeros((B, T, hkv, d)), dv=np.zeros((B, T, hkv, d)))
    for name, q_raw, a, bt, dO, w, pos in (
            ("b", q_base, alpha_b, beta_b, do_base, window, None),
            ("o", q_out, alpha_o, beta_o, do_out, None, out_positions)):
        q_raw = _f64(q_raw)
        dO = _f64(dO)
        A = _f64(a).reshape(hq, d)
        Bt = _f64(bt).reshape(hq, d)
        da = np.zeros((hq, d))
        db = np.zeros((hq, d))
        dq_all = res["dq_base" if name == "b" else "dq_out"]
        for b in range(B):
            for h in range(hq):
                g = _kv_head(h, hq, hkv)
                dqr, dah, dbh, dK, dV = _stream_backward(q_raw[b, :, h], A[h], Bt[h], k[b, :, g],
                                                         v[b, :, g], dO[b, :, h], w, s, pos)
                dq_all[b, :, h] = dqr
                da[h] += dah
                db[h] += dbh
                res["dk"][b, :, g] += dK
                res["dv"][b, :, g] += dV
        res["dalpha_" + name] = da.reshape(-1)
        res["dbeta_" + name] = db.reshape(-1)
    return res
