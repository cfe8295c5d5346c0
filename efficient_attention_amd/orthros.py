"""ctypes binding of liborthros.so (declared in include/orthros.h).

Argument marshalling only: every entry point checks that the torch tensors it is handed have
the shape, dtype, device and layout the C ABI documents, then passes raw device pointers and
the current HIP stream. All arithmetic runs in the library's HIP kernels. If the library is not
built the first call raises; nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "OK", "E_INVALID", "E_UNSUPPORTED", "E_WORKSPACE", "E_LAUNCH",
    "STATUS_CACHE_FULL", "STATUS_BAD_PAGE", "STAGES", "OrthrosError", "Shape", "Affine",
    "PagedKV", "lib", "library_path", "workspace_bytes",
    "make_workspace", "prefill", "prefill_chunk", "prefill_chunk_paged", "decode_step",
    "decode_step_paged", "decode_step_noalloc",
    "paged_write", "forward_pt", "forward_sft", "forward_pt_lse", "backward_workspace_bytes",
    "backward_pt", "forward_sft_lse", "backward_sft_workspace_bytes", "backward_sft",
    "read_device_status", "status_string",
    "timing_begin", "timing_end", "EXPORTED_SYMBOLS",
]

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_LAUNCH = 0, -1, -2, -3, -4
STATUS_CACHE_FULL = 1
STATUS_BAD_PAGE = 2
F32, BF16 = 0, 1
STAGES = ("cache_write", "band", "split_rows", "merge", "append", "rows_f32", "bwd_q", "bwd_kv",
          "bwd_affine")
EXPORTED_SYMBOLS = (
    "orthros_workspace_bytes", "orthros_prefill",
    "orthros_prefill_chunk", "orthros_prefill_chunk_paged", "orthros_decode_step",
    "orthros_decode_step_paged", "orthros_decode_step_noalloc",
    "orthros_paged_write", "orthros_forward_pt", "orthros_forward_sft",
    "orthros_forward_pt_lse", "orthros_backward_workspace_bytes", "orthros_backward_pt",
    "orthros_forward_sft_lse", "orthros_backward_sft_workspace_bytes", "orthros_backward_sft",
    "orthros_read_device_status", "orthros_status_string", "orthros_timing_begin",
    "orthros_timing_end",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class OrthrosError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


class _CShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class _CAffine(ctypes.Structure):
    _fields_ = [("alpha_base", ctypes.c_void_p), ("beta_base", ctypes.c_void_p),
                ("alpha_out", ctypes.c_void_p), ("beta_out", ctypes.c_void_p)]


class _CAffineGrad(ctypes.Structure):
    _fields_ = [("dalpha_base", ctypes.c_void_p), ("dbeta_base", ctypes.c_void_p),
                ("dalpha_out", ctypes.c_void_p), ("dbeta_out", ctypes.c_void_p)]


class _CPagedKV(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("ORTHROS_LIB", os.path.join(_HERE, "liborthros.so"))


def lib() -> ctypes.CDLL:
    """Load liborthros.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sp, ap = ctypes.POINTER(_CShape), ctypes.POINTER(_CAffine)
        L.orthros_workspace_bytes.argtypes = [sp, i64]
        L.orthros_workspace_bytes.restype = sz
        L.orthros_prefill.argtypes = [sp, i64, vp, vp, vp, vp, ap, vp, vp, vp, vp, vp, vp, sz, vp]
        L.orthros_prefill.restype = ctypes.c_int
        L.orthros_decode_step.argtypes = [sp, vp, vp, vp, vp, ap, vp, vp, vp, i64, vp, vp, vp, sz, vp]
        L.orthros_decode_step.restype = ctypes.c_int
        L.orthros_decode_step_noalloc.argtypes = [sp, vp, vp, vp, vp, ap, vp, vp, vp, i64, vp,
                                                  vp, vp, vp]
        L.orthros_decode_step_noalloc.restype = ctypes.c_int
        L.orthros_forward_pt.argtypes = [sp, i64, vp, vp, vp, vp, ap, vp, vp, vp, vp, vp, vp, sz, vp]
        L.orthros_forward_pt.restype = ctypes.c_int
        L.orthros_forward_sft.argtypes = [sp, i64, vp, vp, vp, i64, vp, vp, ap, vp, vp, vp, vp,
                                          vp, vp, sz, vp]
        L.orthros_forward_sft.restype = ctypes.c_int
        L.orthros_prefill_chunk.argtypes = [sp, i64, i64, vp, vp, vp, vp, ap, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
        L.orthros_prefill_chunk.restype = ctypes.c_int
        pp = ctypes.POINTER(_CPagedKV)
        L.orthros_decode_step_paged.argtypes = [sp, vp, vp, vp, vp, ap, pp, vp, i64, vp, vp, vp,
                                                sz, vp]
        L.orthros_decode_step_paged.restype = ctypes.c_int
        L.orthros_prefill_chunk_paged.argtypes = [sp, i64, i64, vp, vp, vp, vp, ap, pp, vp, vp,
                                                  vp, vp, sz, vp]
        L.orthros_prefill_chunk_paged.restype = ctypes.c_int
        L.orthros_paged_write.argtypes = [sp, i64, vp, vp, pp, vp, vp, sz, vp]
        L.orthros_paged_write.restype = ctypes.c_int
        L.orthros_forward_pt_lse.argtypes = [sp, i64, vp, vp, vp, vp, ap, vp, vp, vp, vp, vp, sz,
                                             vp]
        L.orthros_forward_pt_lse.restype = ctypes.c_int
        L.orthros_backward_workspace_bytes.argtypes = [sp, i64]
        L.orthros_backward_workspace_bytes.restype = sz
        L.orthros_backward_pt.argtypes = [sp, i64, vp, vp, vp, vp, ap, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, ctypes.POINTER(_CAffineGrad), vp, sz,
                                          vp]
        L.orthros_backward_pt.restype = ctypes.c_int
        L.orthros_forward_sft_lse.argtypes = [sp, i64, vp, vp, vp, i64, vp, vp, ap, vp, vp, vp,
                                              vp, vp, sz, vp]
        L.orthros_forward_sft_lse.restype = ctypes.c_int
        L.orthros_backward_sft_workspace_bytes.argtypes = [sp, i64, i64]
        L.orthros_backward_sft_workspace_bytes.restype = sz
        L.orthros_backward_sft.argtypes = [sp, i64, vp, vp, vp, i64, vp, vp, ap, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp, ctypes.POINTER(_CAffineGrad),
                                           vp, sz, vp]
        L.orthros_backward_sft.restype = ctypes.c_int
        L.orthros_read_device_status.argtypes = [vp, sz, ctypes.POINTER(i32), ctypes.c_int, vp]
        L.orthros_read_device_status.restype = ctypes.c_int
        L.orthros_status_string.argtypes = [ctypes.c_int]
        L.orthros_status_string.restype = ctypes.c_char_p
        L.orthros_timing_begin.argtypes = []
        L.orthros_timing_begin.restype = ctypes.c_int
        L.orthros_timing_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
        L.orthros_timing_end.restype = ctypes.c_int
        _LIB = L
    return _LIB


def status_string(code: int) -> str:
    return lib().orthros_status_string(int(code)).decode()


@dataclass(frozen=True)
class Shape:
    """Problem shape (the C struct orthros_shape)."""
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    dtype: torch.dtype
    capacity: int
    softmax_scale: float = 0.0

    def c(self) -> _CShape:
        code = {torch.float32: F32, torch.bfloat16: BF16}.get(self.dtype, 99)
        return _CShape(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                       self.window, code, self.capacity, self.softmax_scale, 0)


@dataclass(frozen=True)
class Affine:
    """Scale-offset vectors, fp32 [num_q_heads * head_dim] device tensors."""
    alpha_base: torch.Tensor
    beta_base: torch.Tensor
    alpha_out: torch.Tensor
    beta_out: torch.Tensor

    def c(self, n: int, device) -> _CAffine:
        for t in (self.alpha_base, self.beta_base, self.alpha_out, self.beta_out):
            _check(t, (n,), torch.float32, device, "scale-offset vector")
        return _CAffine(self.alpha_base.data_ptr(), self.beta_base.data_ptr(),
                        self.alpha_out.data_ptr(), self.beta_out.data_ptr())


@dataclass(frozen=True)
class PagedKV:
    """Paged cache (the C struct orthros_paged_kv): k_pages, v_pages [num_pages, H_kv,
    page_size, d] and block_table int32 [batch, max_pages], all on the device."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor

    @property
    def page_size(self) -> int:
        return int(self.k_pages.shape[2])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def c(self, shape: "Shape", device) -> _CPagedKV:
        n, _, ps, _ = self.k_pages.shape
        dims = (n, shape.num_kv_heads, ps, shape.head_dim)
        _check(self.k_pages, dims, shape.dtype, device, "k_pages")
        _check(self.v_pages, dims, shape.dtype, device, "v_pages")
        _check(self.block_table, (shape.batch, self.max_pages), torch.int32, device,
               "block_table")
        return _CPagedKV(self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                         self.block_table.data_ptr(), n, ps, self.max_pages)


def _check(t, shape, dtype, device, what):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{what}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _ptr(t):
    """Device address of an optional tensor (0, i.e. NULL, for None)."""
    return 0 if t is None else t.data_ptr()


def _check_out_row(q_out, o_out, shape, dtype, device):
    """An optional output-stream row: q_out and o_out both given (and checked) or both None."""
    if (q_out is None) != (o_out is None):
        raise ValueError("q_out and o_out must both be given or both be None")
    if q_out is not None:
        _check(q_out, shape, dtype, device, "q_out")
        _check(o_out, shape, dtype, device, "o_out")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _rc(code: int, what: str):
    if code != OK:
        raise OrthrosError(code, what)


def workspace_bytes(shape: Shape, max_rows: int = 1) -> int:
    """orthros_workspace_bytes: max_rows is the most output-stream rows per sequence of one
    call (R for fine-tuning with R response rows, 1 otherwise)."""
    return int(lib().orthros_workspace_bytes(ctypes.byref(shape.c()), int(max_rows)))


def make_workspace(shape: Shape, device, sft_rows: int = 0) -> torch.Tensor:
    """A zero-filled workspace (the status word must start at 0); sft_rows > 0 sizes it for
    orthros_forward_sft with that many response rows."""
    n = workspace_bytes(shape, max(1, sft_rows))
    if n == 0:
        raise OrthrosError(E_INVALID, "workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def prefill(shape: Shape, q_base, q_out, k, v, affine: Affine, cache_k, cache_v, cache_len,
            o_base, o_out, workspace, stream=None):
    """orthros_prefill: base rows over the prompt, one output row at its last token."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    P = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, P, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, 1, Hq, d), dt, dev, "q_out")
    _check(k, (B, P, Hkv, d), dt, dev, "k")
    _check(v, (B, P, Hkv, d), dt, dev, "v")
    _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
    _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, P, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, 1, Hq, d), dt, dev, "o_out")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_prefill(
        ctypes.byref(shape.c()), P, q_base.data_ptr(), q_out.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(aff), cache_k.data_ptr(), cache_v.data_ptr(),
        cache_len.data_ptr(), o_base.data_ptr(), o_out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(stream))
    _rc(rc, "orthros_prefill")


def prefill_chunk(shape: Shape, past_len: int, q_base, q_out, k, v, affine: Affine, cache_k,
                  cache_v, cache_len, o_base, o_out, workspace, stream=None):
    """orthros_prefill_chunk: C more prompt tokens after past_len already cached ones. q_out
    and o_out may both be None: no output-stream row (a chunk before the prompt's last)."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    C = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, C, Hq, d), dt, dev, "q_base")
    _check_out_row(q_out, o_out, (B, 1, Hq, d), dt, dev)
    _check(k, (B, C, Hkv, d), dt, dev, "k")
    _check(v, (B, C, Hkv, d), dt, dev, "v")
    _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
    _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, C, Hq, d), dt, dev, "o_base")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_prefill_chunk(
        ctypes.byref(shape.c()), int(past_len), C, q_base.data_ptr(), _ptr(q_out),
        k.data_ptr(), v.data_ptr(), ctypes.byref(aff), cache_k.data_ptr(), cache_v.data_ptr(),
        cache_len.data_ptr(), o_base.data_ptr(), _ptr(o_out), workspace.data_ptr(),
        workspace.numel(), _stream(stream))
    _rc(rc, "orthros_prefill_chunk")


def decode_step(shape: Shape, q_base, q_out, k_new, v_new, affine: Affine, cache_k, cache_v,
                cache_len, max_len_hint: int, o_base, o_out, workspace, stream=None):
    """orthros_decode_step: one decoupled base/output pair per sequence."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, Hq, d), dt, dev, "q_out")
    _check(k_new, (B, Hkv, d), dt, dev, "k_new")
    _check(v_new, (B, Hkv, d), dt, dev, "v_new")
    _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
    _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, Hq, d), dt, dev, "o_out")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_decode_step(
        ctypes.byref(shape.c()), q_base.data_ptr(), q_out.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), ctypes.byref(aff), cache_k.data_ptr(), cache_v.data_ptr(),
        cache_len.data_ptr(), int(max_len_hint), o_base.data_ptr(), o_out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _rc(rc, "orthros_decode_step")


def decode_step_noalloc(shape: Shape, q_base, q_out, k_new, v_new, affine: Affine, cache_k,
                        cache_v, cache_len, max_len_hint: int, o_base, o_out, device_status,
                        stream=None):
    """orthros_decode_step_noalloc: orthros_decode_step without a workspace (the split partials
    live in the library's own device array); status bits are OR-ed into device_status."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, Hq, d), dt, dev, "q_out")
    _check(k_new, (B, Hkv, d), dt, dev, "k_new")
    _check(v_new, (B, Hkv, d), dt, dev, "v_new")
    _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
    _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, Hq, d), dt, dev, "o_out")
    _check(device_status, (1,), torch.int32, dev, "device_status")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_decode_step_noalloc(
        ctypes.byref(shape.c()), q_base.data_ptr(), q_out.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), ctypes.byref(aff), cache_k.data_ptr(), cache_v.data_ptr(),
        cache_len.data_ptr(), int(max_len_hint), o_base.data_ptr(), o_out.data_ptr(),
        device_status.data_ptr(), _stream(stream))
    _rc(rc, "orthros_decode_step_noalloc")


def decode_step_paged(shape: Shape, q_base, q_out, k_new, v_new, affine: Affine,
                      cache: PagedKV, cache_len, max_len_hint: int, o_base, o_out, workspace,
                      stream=None):
    """orthros_decode_step_paged: the decode pair over a paged cache."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, Hq, d), dt, dev, "q_out")
    _check(k_new, (B, Hkv, d), dt, dev, "k_new")
    _check(v_new, (B, Hkv, d), dt, dev, "v_new")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, Hq, d), dt, dev, "o_out")
    aff = affine.c(Hq * d, dev)
    pc = cache.c(shape, dev)
    rc = lib().orthros_decode_step_paged(
        ctypes.byref(shape.c()), q_base.data_ptr(), q_out.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), ctypes.byref(aff), ctypes.byref(pc), cache_len.data_ptr(),
        int(max_len_hint), o_base.data_ptr(), o_out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(stream))
    _rc(rc, "orthros_decode_step_paged")


def prefill_chunk_paged(shape: Shape, past_len: int, q_base, q_out, k, v, affine: Affine,
                        cache: PagedKV, cache_len, o_base, o_out, workspace, stream=None):
    """orthros_prefill_chunk_paged: C more prompt tokens into a paged cache (q_out and o_out
    may both be None, as for prefill_chunk)."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    C = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, C, Hq, d), dt, dev, "q_base")
    _check_out_row(q_out, o_out, (B, 1, Hq, d), dt, dev)
    _check(k, (B, C, Hkv, d), dt, dev, "k")
    _check(v, (B, C, Hkv, d), dt, dev, "v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    _check(o_base, (B, C, Hq, d), dt, dev, "o_base")
    aff = affine.c(Hq * d, dev)
    pc = cache.c(shape, dev)
    rc = lib().orthros_prefill_chunk_paged(
        ctypes.byref(shape.c()), int(past_len), C, q_base.data_ptr(), _ptr(q_out),
        k.data_ptr(), v.data_ptr(), ctypes.byref(aff), ctypes.byref(pc), cache_len.data_ptr(),
        o_base.data_ptr(), _ptr(o_out), workspace.data_ptr(), workspace.numel(),
        _stream(stream))
    _rc(rc, "orthros_prefill_chunk_paged")


def paged_write(shape: Shape, k, v, cache: PagedKV, cache_len, workspace, stream=None):
    """orthros_paged_write: append k, v [B, T, H_kv, d] to a paged cache."""
    B, Hkv, d = shape.batch, shape.num_kv_heads, shape.head_dim
    T = k.shape[1]
    dev, dt = k.device, shape.dtype
    _check(k, (B, T, Hkv, d), dt, dev, "k")
    _check(v, (B, T, Hkv, d), dt, dev, "v")
    _check(cache_len, (B,), torch.int32, dev, "cache_len")
    pc = cache.c(shape, dev)
    rc = lib().orthros_paged_write(ctypes.byref(shape.c()), T, k.data_ptr(), v.data_ptr(),
                                   ctypes.byref(pc), cache_len.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), _stream(stream))
    _rc(rc, "orthros_paged_write")


def forward_pt(shape: Shape, q_base, q_out, k, v, affine: Affine, o_base, o_out, workspace,
               cache_k=None, cache_v=None, cache_len=None, stream=None):
    """orthros_forward_pt: every position duplicated (pre-training regime)."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, T, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, T, Hq, d), dt, dev, "q_out")
    _check(k, (B, T, Hkv, d), dt, dev, "k")
    _check(v, (B, T, Hkv, d), dt, dev, "v")
    _check(o_base, (B, T, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, T, Hq, d), dt, dev, "o_out")
    ck = cv = cl = 0
    if cache_k is not None or cache_v is not None or cache_len is not None:
        _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
        _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
        _check(cache_len, (B,), torch.int32, dev, "cache_len")
        ck, cv, cl = cache_k.data_ptr(), cache_v.data_ptr(), cache_len.data_ptr()
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_forward_pt(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(aff), ck or None, cv or None, cl or None, o_base.data_ptr(),
        o_out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream))
    _rc(rc, "orthros_forward_pt")


def forward_sft(shape: Shape, q_base, q_out, out_pos, k, v, affine: Affine, o_base, o_out,
                workspace, cache_k=None, cache_v=None, cache_len=None, stream=None):
    """orthros_forward_sft: base rows everywhere, output rows at the response positions."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T, R = q_base.shape[1], q_out.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, T, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, R, Hq, d), dt, dev, "q_out")
    _check(out_pos, (R,), torch.int32, dev, "out_pos")
    _check(k, (B, T, Hkv, d), dt, dev, "k")
    _check(v, (B, T, Hkv, d), dt, dev, "v")
    _check(o_base, (B, T, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, R, Hq, d), dt, dev, "o_out")
    ck = cv = cl = 0
    if cache_k is not None or cache_v is not None or cache_len is not None:
        _check(cache_k, (B, Hkv, shape.capacity, d), dt, dev, "cache_k")
        _check(cache_v, (B, Hkv, shape.capacity, d), dt, dev, "cache_v")
        _check(cache_len, (B,), torch.int32, dev, "cache_len")
        ck, cv, cl = cache_k.data_ptr(), cache_v.data_ptr(), cache_len.data_ptr()
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_forward_sft(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), out_pos.data_ptr(), R,
        k.data_ptr(), v.data_ptr(), ctypes.byref(aff), ck or None, cv or None, cl or None,
        o_base.data_ptr(), o_out.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream(stream))
    _rc(rc, "orthros_forward_sft")


def forward_pt_lse(shape: Shape, q_base, q_out, k, v, affine: Affine, o_base, o_out, lse_base,
                   lse_out, workspace, stream=None):
    """orthros_forward_pt_lse: the pre-training forward plus per-row log-sum-exp."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, T, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, T, Hq, d), dt, dev, "q_out")
    _check(k, (B, T, Hkv, d), dt, dev, "k")
    _check(v, (B, T, Hkv, d), dt, dev, "v")
    _check(o_base, (B, T, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, T, Hq, d), dt, dev, "o_out")
    _check(lse_base, (B, Hq, T), torch.float32, dev, "lse_base")
    _check(lse_out, (B, Hq, T), torch.float32, dev, "lse_out")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_forward_pt_lse(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(aff), o_base.data_ptr(), o_out.data_ptr(),
        lse_base.data_ptr(), lse_out.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream(stream))
    _rc(rc, "orthros_forward_pt_lse")


def backward_workspace_bytes(shape: Shape, T: int) -> int:
    return int(lib().orthros_backward_workspace_bytes(ctypes.byref(shape.c()), int(T)))


def backward_pt(shape: Shape, q_base, q_out, k, v, affine: Affine, o_base, o_out, lse_base,
                lse_out, do_base, do_out, dq_base, dq_out, dk, dv, dgrad, workspace,
                stream=None):
    """orthros_backward_pt. dgrad: (dalpha_base, dbeta_base, dalpha_out, dbeta_out), fp32
    [num_q_heads * head_dim] device tensors (outputs)."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T = q_base.shape[1]
    dev, dt = q_base.device, shape.dtype
    for t, n in ((q_base, "q_base"), (q_out, "q_out"), (o_base, "o_base"), (o_out, "o_out"),
                 (do_base, "do_base"), (do_out, "do_out"), (dq_base, "dq_base"),
                 (dq_out, "dq_out")):
        _check(t, (B, T, Hq, d), dt, dev, n)
    for t, n in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _check(t, (B, T, Hkv, d), dt, dev, n)
    _check(lse_base, (B, Hq, T), torch.float32, dev, "lse_base")
    _check(lse_out, (B, Hq, T), torch.float32, dev, "lse_out")
    for t in dgrad:
        _check(t, (Hq * d,), torch.float32, dev, "scale-offset gradient")
    aff = affine.c(Hq * d, dev)
    g = _CAffineGrad(*(t.data_ptr() for t in dgrad))
    rc = lib().orthros_backward_pt(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(aff), o_base.data_ptr(), o_out.data_ptr(),
        lse_base.data_ptr(), lse_out.data_ptr(), do_base.data_ptr(), do_out.data_ptr(),
        dq_base.data_ptr(), dq_out.data_ptr(), dk.data_ptr(), dv.data_ptr(), ctypes.byref(g),
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _rc(rc, "orthros_backward_pt")


def forward_sft_lse(shape: Shape, q_base, q_out, out_pos, k, v, affine: Affine, o_base, o_out,
                    lse_base, lse_out, workspace, stream=None):
    """orthros_forward_sft_lse: the fine-tuning forward plus per-row log-sum-exp."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T, R = q_base.shape[1], q_out.shape[1]
    dev, dt = q_base.device, shape.dtype
    _check(q_base, (B, T, Hq, d), dt, dev, "q_base")
    _check(q_out, (B, R, Hq, d), dt, dev, "q_out")
    _check(out_pos, (R,), torch.int32, dev, "out_pos")
    _check(k, (B, T, Hkv, d), dt, dev, "k")
    _check(v, (B, T, Hkv, d), dt, dev, "v")
    _check(o_base, (B, T, Hq, d), dt, dev, "o_base")
    _check(o_out, (B, R, Hq, d), dt, dev, "o_out")
    _check(lse_base, (B, Hq, T), torch.float32, dev, "lse_base")
    _check(lse_out, (B, Hq, R), torch.float32, dev, "lse_out")
    aff = affine.c(Hq * d, dev)
    rc = lib().orthros_forward_sft_lse(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), out_pos.data_ptr(), R,
        k.data_ptr(), v.data_ptr(), ctypes.byref(aff), o_base.data_ptr(), o_out.data_ptr(),
        lse_base.data_ptr(), lse_out.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream(stream))
    _rc(rc, "orthros_forward_sft_lse")


def backward_sft_workspace_bytes(shape: Shape, T: int, R: int) -> int:
    return int(lib().orthros_backward_sft_workspace_bytes(ctypes.byref(shape.c()), int(T),
                                                          int(R)))


def backward_sft(shape: Shape, q_base, q_out, out_pos, k, v, affine: Affine, o_base, o_out,
                 lse_base, lse_out, do_base, do_out, dq_base, dq_out, dk, dv, dgrad, workspace,
                 stream=None):
    """orthros_backward_sft: gradients with output rows only at the response positions."""
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    T, R = q_base.shape[1], q_out.shape[1]
    dev, dt = q_base.device, shape.dtype
    for t, n in ((q_base, "q_base"), (o_base, "o_base"), (do_base, "do_base"),
                 (dq_base, "dq_base")):
        _check(t, (B, T, Hq, d), dt, dev, n)
    for t, n in ((q_out, "q_out"), (o_out, "o_out"), (do_out, "do_out"), (dq_out, "dq_out")):
        _check(t, (B, R, Hq, d), dt, dev, n)
    for t, n in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _check(t, (B, T, Hkv, d), dt, dev, n)
    _check(out_pos, (R,), torch.int32, dev, "out_pos")
    _check(lse_base, (B, Hq, T), torch.float32, dev, "lse_base")
    _check(lse_out, (B, Hq, R), torch.float32, dev, "lse_out")
    for t in dgrad:
        _check(t, (Hq * d,), torch.float32, dev, "scale-offset gradient")
    aff = affine.c(Hq * d, dev)
    g = _CAffineGrad(*(t.data_ptr() for t in dgrad))
    rc = lib().orthros_backward_sft(
        ctypes.byref(shape.c()), T, q_base.data_ptr(), q_out.data_ptr(), out_pos.data_ptr(), R,
        k.data_ptr(), v.data_ptr(), ctypes.byref(aff), o_base.data_ptr(), o_out.data_ptr(),
        lse_base.data_ptr(), lse_out.data_ptr(), do_base.data_ptr(), do_out.data_ptr(),
        dq_base.data_ptr(), dq_out.data_ptr(), dk.data_ptr(), dv.data_ptr(), ctypes.byref(g),
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _rc(rc, "orthros_backward_sft")


def read_device_status(workspace, clear: bool = False, stream=None) -> int:
    out = ctypes.c_int32(0)
    rc = lib().orthros_read_device_status(workspace.data_ptr(), workspace.numel(),
                                          ctypes.byref(out), int(bool(clear)), _stream(stream))
    _rc(rc, "orthros_read_device_status")
    return int(out.value)


def timing_begin():
    _rc(lib().orthros_timing_begin(), "orthros_timing_begin")


def timing_end():
    """Returns {stage: (total_ms, launches)} for the calls since timing_begin()."""
    ms = (ctypes.c_double * len(STAGES))()
    n = (ctypes.c_int64 * len(STAGES))()
    _rc(lib().orthros_timing_end(ms, n), "orthros_timing_end")
    return {name: (ms[i], int(n[i])) for i, name in enumerate(STAGES)}
