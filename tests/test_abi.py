"""CPU checks of the C ABI: the library loads, exports every function include/orthros.h
declares, and rejects bad arguments before enqueuing anything.

Every call below carries exactly one defect, so it returns at validation and never reaches a
kernel launch (fake pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

from efficient_attention_amd import orthros as ox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthros.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ox.library_path()),
                                reason="liborthros.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(orthros_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert header_functions() == sorted(ox.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ox.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (orthros_[a-z_]+)$", out, flags=re.M))
    missing = set(header_functions()) - exported
    assert not missing, f"declared but not exported: {missing}"
    L = ox.lib()
    for name in header_functions():
        assert hasattr(L, name)


def test_missing_library_fails_loudly(tmp_path):
    code = ("import os; os.environ['ORTHROS_LIB'] = %r\n"
            "from efficient_attention_amd import orthros as ox\n"
            "try:\n    ox.lib()\nexcept RuntimeError as e:\n    print('raised', e)\n" %
            str(tmp_path / "nope.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in r.stdout


def _shape(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, window=16, dtype=1,
                capacity=1024, softmax_scale=0.0, reserved=0)
    base.update(kw)
    return ox._CShape(**{k: base[k] for k, _ in ox._CShape._fields_})


FAKE = 1 << 20  # 16-byte aligned, never dereferenced


def _aff(**kw):
    a = dict(alpha_base=FAKE, beta_base=FAKE, alpha_out=FAKE, beta_out=FAKE)
    a.update(kw)
    return ox._CAffine(**a)


def _prefill(shape, P=64, aff=None, ws_bytes=None, **ptrs):
    p = dict(q_base=FAKE, q_out=FAKE, k=FAKE, v=FAKE, cache_k=FAKE, cache_v=FAKE, cache_len=FAKE,
             o_base=FAKE, o_out=FAKE, ws=FAKE)
    p.update(ptrs)
    L = ox.lib()
    wsb = L.orthros_workspace_bytes(ctypes.byref(shape), 1) if ws_bytes is None else ws_bytes
    return L.orthros_prefill(ctypes.byref(shape), P, p["q_base"], p["q_out"], p["k"], p["v"],
                             ctypes.byref(aff or _aff()), p["cache_k"], p["cache_v"],
                             p["cache_len"], p["o_base"], p["o_out"], p["ws"], wsb, None)


def test_workspace_bytes():
    L = ox.lib()
    n = L.orthros_workspace_bytes(ctypes.byref(_shape()), 1)
    # status + (max, sum) + d partials for B * Hq * 2 rows * 64 splits
    assert n >= 2 * 8 * 2 * 64 * (128 + 2) * 4
    assert L.orthros_workspace_bytes(ctypes.byref(_shape(head_dim=96)), 1) == 0
    assert L.orthros_workspace_bytes(None, 1) == 0


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, ox.E_INVALID), ("num_q_heads", 0, ox.E_INVALID),
    ("num_kv_heads", 3, ox.E_INVALID), ("window", 0, ox.E_INVALID),
    ("capacity", 0, ox.E_INVALID), ("reserved", 1, ox.E_INVALID),
    ("head_dim", 96, ox.E_UNSUPPORTED), ("dtype", 7, ox.E_UNSUPPORTED),
])
def test_prefill_rejects_bad_shape(field, value, code):
    assert _prefill(_shape(**{field: value}), ws_bytes=1 << 30) == code


@pytest.mark.parametrize("name", ["q_base", "q_out", "k", "v", "cache_k", "cache_v",
                                  "cache_len", "o_base", "o_out"])
def test_prefill_rejects_null_and_misaligned(name):
    assert _prefill(_shape(), **{name: None}) == ox.E_INVALID
    assert _prefill(_shape(), **{name: FAKE + 8}) == ox.E_INVALID


def test_prefill_rejects_bad_affine_workspace_capacity_and_length():
    assert _prefill(_shape(), aff=_aff(beta_out=None)) == ox.E_INVALID
    assert _prefill(_shape(), ws=None) == ox.E_WORKSPACE
    assert _prefill(_shape(), ws_bytes=100) == ox.E_WORKSPACE
    assert _prefill(_shape(capacity=63), P=64) == ox.E_INVALID
    assert _prefill(_shape(), P=0) == ox.E_INVALID


def test_decode_and_pt_reject_bad_arguments():
    L = ox.lib()
    s = _shape()
    wsb = L.orthros_workspace_bytes(ctypes.byref(s), 1)
    F = FAKE
    rc = L.orthros_decode_step(ctypes.byref(s), F, F, None, F, ctypes.byref(_aff()), F, F, F, 10,
                               F, F, F, wsb, None)
    assert rc == ox.E_INVALID
    rc = L.orthros_decode_step(ctypes.byref(s), F, F, F, F, ctypes.byref(_aff()), F, F, F, -1,
                               F, F, F, wsb, None)
    assert rc == ox.E_INVALID
    rc = L.orthros_decode_step(ctypes.byref(s), F, F, F, F, ctypes.byref(_aff()), F, F, F, 10,
                               F, F, F, wsb - 1, None)
    assert rc == ox.E_WORKSPACE
    # pre-training: the cache is all-or-nothing
    rc = L.orthros_forward_pt(ctypes.byref(s), 64, F, F, F, F, ctypes.byref(_aff()), F, None, None,
                              F, F, F, wsb, None)
    assert rc == ox.E_INVALID
    rc = L.orthros_forward_pt(ctypes.byref(_shape(capacity=32)), 64, F, F, F, F,
                              ctypes.byref(_aff()), F, F, F, F, F, F, wsb, None)
    assert rc == ox.E_INVALID
    rc = L.orthros_forward_pt(ctypes.byref(_shape(head_dim=32)), 64, F, F, F, F,
                              ctypes.byref(_aff()), None, None, None, F, F, F, wsb, None)
    assert rc == ox.E_UNSUPPORTED


def test_status_strings():
    for code in (ox.OK, ox.E_INVALID, ox.E_UNSUPPORTED, ox.E_WORKSPACE, 
                 ox.E_LAUNCH):
        assert ox.status_string(code) not in ("", "unknown status")
    assert ox.status_string(12345) == "unknown status"


def test_read_status_rejects_null():
    out = ctypes.c_int32(0)
    assert ox.lib().orthros_read_device_status(None, 4096, ctypes.byref(out), 0, None) == ox.E_INVALID


def test_sft_workspace_bytes():
    L = ox.lib()
    s = _shape()
    base = L.orthros_workspace_bytes(ctypes.byref(s), 1)
    assert L.orthros_workspace_bytes(ctypes.byref(s), 1) == base
    # up to 16 response rows use split-key rows: one partial row per (head, response row)
    assert L.orthros_workspace_bytes(ctypes.byref(s), 16) > base
    assert L.orthros_workspace_bytes(ctypes.byref(s), 17) == base  # banded path: no partials
    assert L.orthros_workspace_bytes(ctypes.byref(s), 0) == 0
    assert L.orthros_workspace_bytes(ctypes.byref(_shape(head_dim=96)), 4) == 0


def _sft(shape, T=64, R=4, ws_bytes=None, aff=None, **ptrs):
    p = dict(q_base=FAKE, q_out=FAKE, pos=FAKE, k=FAKE, v=FAKE, cache_k=None, cache_v=None,
             cache_len=None, o_base=FAKE, o_out=FAKE, ws=FAKE)
    p.update(ptrs)
    L = ox.lib()
    wsb = L.orthros_workspace_bytes(ctypes.byref(shape), max(R, 1)) if ws_bytes is None else ws_bytes
    return L.orthros_forward_sft(ctypes.byref(shape), T, p["q_base"], p["q_out"], p["pos"], R,
                                 p["k"], p["v"], ctypes.byref(aff or _aff()), p["cache_k"],
                                 p["cache_v"], p["cache_len"], p["o_base"], p["o_out"], p["ws"],
                                 wsb, None)


@pytest.mark.parametrize("name", ["q_base", "q_out", "pos", "k", "v", "o_base", "o_out"])
def test_sft_rejects_null_pointers(name):
    assert _sft(_shape(), **{name: None}) == ox.E_INVALID


def test_sft_rejects_bad_arguments():
    assert _sft(_shape(), pos=FAKE + 2) == ox.E_INVALID        # positions must be int32-aligned
    assert _sft(_shape(), R=0) == ox.E_INVALID
    assert _sft(_shape(), T=0) == ox.E_INVALID
    assert _sft(_shape(), R=8, ws_bytes=ox.lib().orthros_workspace_bytes(ctypes.byref(_shape()), 1)) \
        == ox.E_WORKSPACE                                        # 8 rows need the larger workspace
    assert _sft(_shape(), cache_k=FAKE) == ox.E_INVALID          # cache is all-or-nothing
    assert _sft(_shape(capacity=32), cache_k=FAKE, cache_v=FAKE, cache_len=FAKE) == ox.E_INVALID
    assert _sft(_shape(head_dim=48)) == ox.E_UNSUPPORTED
    assert _sft(_shape(), aff=_aff(alpha_out=None)) == ox.E_INVALID


def _chunk(shape, past=100, C=64, ws_bytes=None, **ptrs):
    p = dict(q_base=FAKE, q_out=FAKE, k=FAKE, v=FAKE, cache_k=FAKE, cache_v=FAKE, cache_len=FAKE,
             o_base=FAKE, o_out=FAKE, ws=FAKE)
    p.update(ptrs)
    L = ox.lib()
    wsb = L.orthros_workspace_bytes(ctypes.byref(shape), 1) if ws_bytes is None else ws_bytes
    return L.orthros_prefill_chunk(ctypes.byref(shape), past, C, p["q_base"], p["q_out"], p["k"],
                                   p["v"], ctypes.byref(_aff()), p["cache_k"], p["cache_v"],
                                   p["cache_len"], p["o_base"], p["o_out"], p["ws"], wsb, None)


@pytest.mark.parametrize("name", ["q_base", "q_out", "k", "v", "cache_k", "cache_v",
                                  "cache_len", "o_base", "o_out"])
def test_prefill_chunk_rejects_null_and_misaligned(name):
    assert _chunk(_shape(), **{name: None}) == ox.E_INVALID
    assert _chunk(_shape(), **{name: FAKE + 4}) == ox.E_INVALID


def test_prefill_chunk_output_row_is_both_or_neither():
    # q_out and o_out may both be NULL (no output row); one of them alone is invalid, and with
    # both NULL the other arguments are still checked
    assert _chunk(_shape(), q_out=None) == ox.E_INVALID
    assert _chunk(_shape(), o_out=None) == ox.E_INVALID
    assert _chunk(_shape(), q_out=None, o_out=None, past=-1) == ox.E_INVALID
    assert _chunk(_shape(), q_out=None, o_out=None, k=None) == ox.E_INVALID
    assert _chunk(_shape(), q_out=None, o_out=None, o_base=FAKE + 4) == ox.E_INVALID
    assert _chunk(_shape(), q_out=None, o_out=None, ws_bytes=64) == ox.E_WORKSPACE
    with pytest.raises(ValueError):
        ox._check_out_row(None, torch.zeros(1), (1,), torch.float32, torch.device("cpu"))


def test_prefill_chunk_rejects_bad_lengths_and_workspace():
    assert _chunk(_shape(), past=-1) == ox.E_INVALID
    assert _chunk(_shape(), C=0) == ox.E_INVALID
    assert _chunk(_shape(capacity=163), past=100, C=64) == ox.E_INVALID
    assert _chunk(_shape(capacity=164), past=100, C=64, ws=None) == ox.E_WORKSPACE
    assert _chunk(_shape(), ws_bytes=64) == ox.E_WORKSPACE


def _paged(**kw):
    c = dict(k_pages=FAKE, v_pages=FAKE, block_table=FAKE, num_pages=100, page_size=64,
             max_pages=16)
    c.update(kw)
    return ox._CPagedKV(**c)


def _decode_paged(shape, cache=None, hint=100, ws_bytes=None, **ptrs):
    p = dict(q_base=FAKE, q_out=FAKE, k_new=FAKE, v_new=FAKE, cache_len=FAKE, o_base=FAKE,
             o_out=FAKE, ws=FAKE)
    p.update(ptrs)
    L = ox.lib()
    wsb = L.orthros_workspace_bytes(ctypes.byref(shape), 1) if ws_bytes is None else ws_bytes
    c = cache if cache is not None else _paged()
    return L.orthros_decode_step_paged(ctypes.byref(shape), p["q_base"], p["q_out"], p["k_new"],
                                       p["v_new"], ctypes.byref(_aff()), ctypes.byref(c),
                                       p["cache_len"], hint, p["o_base"], p["o_out"], p["ws"],
                                       wsb, None)


def _paged_write(shape, T=8, cache=None, ws_bytes=None, **ptrs):
    p = dict(k=FAKE, v=FAKE, cache_len=FAKE, ws=FAKE)
    p.update(ptrs)
    L = ox.lib()
    wsb = L.orthros_workspace_bytes(ctypes.byref(shape), 1) if ws_bytes is None else ws_bytes
    c = cache if cache is not None else _paged()
    return L.orthros_paged_write(ctypes.byref(shape), T, p["k"], p["v"], ctypes.byref(c),
                                 p["cache_len"], p["ws"], wsb, None)


@pytest.mark.parametrize("name", ["q_base", "q_out", "k_new", "v_new", "cache_len", "o_base",
                                  "o_out"])
def test_decode_paged_rejects_null_and_misaligned(name):
    assert _decode_paged(_shape(), **{name: None}) == ox.E_INVALID
    assert _decode_paged(_shape(), **{name: FAKE + 4}) == ox.E_INVALID


@pytest.mark.parametrize("bad", [dict(k_pages=None), dict(v_pages=FAKE + 8),
                                 dict(block_table=None), dict(num_pages=0),
                                 dict(num_pages=1 << 31), dict(max_pages=0),
                                 dict(page_size=0), dict(page_size=48),  # not a power of two
                                 dict(page_size=32),                      # capacity 512 != 1024
                                 dict(max_pages=17)])                     # capacity 1088
def test_paged_cache_descriptor_is_validated(bad):
    shape = _shape()  # capacity 1024 = 16 pages x 64
    assert _decode_paged(shape, cache=_paged(**bad)) == ox.E_INVALID
    assert _paged_write(shape, cache=_paged(**bad)) == ox.E_INVALID


def test_paged_calls_reject_bad_shape_lengths_and_workspace():
    L = ox.lib()
    assert L.orthros_decode_step_paged(ctypes.byref(_shape()), FAKE, FAKE, FAKE, FAKE,
                                       ctypes.byref(_aff()), None, FAKE, 1, FAKE, FAKE, FAKE,
                                       1 << 30, None) == ox.E_INVALID
    assert _decode_paged(_shape(head_dim=96)) == ox.E_UNSUPPORTED
    assert _decode_paged(_shape(), hint=-1) == ox.E_INVALID
    assert _decode_paged(_shape(), ws_bytes=100) == ox.E_WORKSPACE
    assert _decode_paged(_shape(), ws=None) == ox.E_WORKSPACE
    assert _paged_write(_shape(), T=0) == ox.E_INVALID
    assert _paged_write(_shape(), k=None) == ox.E_INVALID
    assert _paged_write(_shape(), ws_bytes=16) == ox.E_WORKSPACE


def test_paged_prefill_chunk_validation():
    L = ox.lib()
    shape = _shape()  # bf16, capacity 1024

    def call(cache, past=0, C=16):
        return L.orthros_prefill_chunk_paged(
            ctypes.byref(shape), past, C, FAKE, FAKE, FAKE, FAKE, ctypes.byref(_aff()),
            ctypes.byref(cache), FAKE, FAKE, FAKE, FAKE,
            L.orthros_workspace_bytes(ctypes.byref(shape), 1), None)
    # the banded kernel reads one table entry per 64-key tile: bf16 needs pages of >= 64 rows
    assert call(_paged(page_size=32, max_pages=32)) == ox.E_UNSUPPORTED
    assert call(_paged(page_size=48)) == ox.E_INVALID
    assert call(_paged(), past=-1) == ox.E_INVALID
    assert call(_paged(), past=1020, C=8) == ox.E_INVALID


def test_error_codes_match_the_header():
    text = open(HEADER).read()
    codes = dict(re.findall(r"ORTHROS_(OK|E_[A-Z]+)\s*=\s*(-?\d+)", text))
    assert {k: int(v) for k, v in codes.items()} == dict(
        OK=ox.OK, E_INVALID=ox.E_INVALID, E_UNSUPPORTED=ox.E_UNSUPPORTED,
        E_WORKSPACE=ox.E_WORKSPACE, E_LAUNCH=ox.E_LAUNCH)
    assert ox.E_LAUNCH == -4 and ox.E_INVALID == -1


def test_read_status_checks_its_arguments():
    L = ox.lib()
    out = ctypes.c_int32(0)
    # the workspace must hold the 256-byte status block; the host pointer must be set
    assert L.orthros_read_device_status(FAKE, 100, ctypes.byref(out), 0, None) == ox.E_INVALID
    assert L.orthros_read_device_status(FAKE, 4096, None, 1, None) == ox.E_INVALID


# Distinct, far-apart fake addresses so that only the overlaps a test plants exist.
def _addr(i):
    return (1 << 36) + (i << 30)


def _prefill_at(shape, P, k, v, cache_k, cache_v):
    L = ox.lib()
    return L.orthros_prefill(ctypes.byref(shape), P, _addr(1), _addr(2), k, v,
                             ctypes.byref(_aff()), cache_k, cache_v, _addr(3), _addr(4),
                             _addr(5), _addr(6), L.orthros_workspace_bytes(ctypes.byref(shape), 1),
                             None)


def test_keys_overlapping_the_cache_are_rejected():
    ck, cv = _addr(10), _addr(20)
    one = _shape(batch=1, num_q_heads=4, num_kv_heads=1, capacity=1024)
    # k inside the cache but not at its rows 0 .. P-1, or v inside the key cache
    assert _prefill_at(one, 64, ck + 256, cv, ck, cv) == ox.E_INVALID
    assert _prefill_at(one, 64, _addr(30), ck + 4096, ck, cv) == ox.E_INVALID
    # with two kv heads the layouts differ: k == cache_k is an overlap, not the cache rows
    two = _shape(batch=1, num_q_heads=4, num_kv_heads=2, capacity=1024)
    assert _prefill_at(two, 64, ck, cv, ck, cv) == ox.E_INVALID
    # two sequences in one kv head coincide only when capacity == P
    assert _prefill_at(_shape(batch=2, num_q_heads=4, num_kv_heads=1, capacity=1024), 64,
                       ck, cv, ck, cv) == ox.E_INVALID
    L = ox.lib()
    # a chunk's rows start at past_len: k == cache_k (row 0) overlaps rows 0 .. past_len - 1
    assert L.orthros_prefill_chunk(ctypes.byref(one), 100, 64, _addr(1), _addr(2), ck, cv,
                                   ctypes.byref(_aff()), ck, cv, _addr(3), _addr(4), _addr(5),
                                   _addr(6), L.orthros_workspace_bytes(ctypes.byref(one), 1),
                                   None) == ox.E_INVALID


def test_keys_overlapping_a_page_pool_are_rejected():
    pool = _paged(k_pages=_addr(10), v_pages=_addr(20))
    shape = _shape()
    assert _paged_write(shape, cache=pool, k=_addr(10) + 1024, v=_addr(30), cache_len=_addr(31),
                        ws=_addr(32)) == ox.E_INVALID
    assert _paged_write(shape, cache=pool, k=_addr(30), v=_addr(20), cache_len=_addr(31),
                        ws=_addr(32)) == ox.E_INVALID


def test_noalloc_decode_rejects_steps_beyond_its_scratch():
    L = ox.lib()
    F = FAKE
    dst = _addr(40)
    # 64 sequences x 128 query heads: 2 x 64 x 128 rows x (128 + 2) floats > 8 MiB at one split
    big = _shape(batch=64, num_q_heads=128, num_kv_heads=8, capacity=4096)
    assert L.orthros_decode_step_noalloc(ctypes.byref(big), F, F, F, F, ctypes.byref(_aff()),
                                         F, F, F, 100, F, F, dst, None) == ox.E_WORKSPACE
    s = _shape()
    assert L.orthros_decode_step_noalloc(ctypes.byref(s), F, F, F, F, ctypes.byref(_aff()),
                                         F, F, F, 100, F, F, None, None) == ox.E_INVALID
    assert L.orthros_decode_step_noalloc(ctypes.byref(s), F, F, F, F, ctypes.byref(_aff()),
                                         F, F, F, -1, F, F, dst, None) == ox.E_INVALID
