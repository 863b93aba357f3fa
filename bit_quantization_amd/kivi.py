"""Python binding of ``libkivi.so`` (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks that tensors live on the GPU with the expected
dtype and contiguity, passes their device pointers and the current HIP stream, and
turns a non-OK status into an exception carrying ``kivi_last_error()``.  PyTorch
provides device memory and streams only.

If the library is missing, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KIVI_LIBRARY names another build of the same library (the host-sanitized build the CPU
# tests run the ABI checks under); by default the in-tree libkivi.so
LIB_PATH = os.environ.get("KIVI_LIBRARY") or os.path.join(_HERE, "libkivi.so")

STATUS = {0: "KIVI_OK", 1: "KIVI_ERR_ARG", 2: "KIVI_ERR_UNSUPPORTED", 3: "KIVI_ERR_CAPACITY",
          4: "KIVI_ERR_ALIGN", 5: "KIVI_ERR_WORKSPACE", 6: "KIVI_ERR_DEVICE"}

EXPORTS = ("kivi_cache_sizes", "kivi_quantize_k", "kivi_quantize_v", "kivi_append_flush",
           "kivi_decode_workspace_bytes", "kivi_decode_attn", "kivi_decode_attn_split",
           "kivi_append_decode", "kivi_append_decode_noalloc", "kivi_paged_cache_sizes",
           "kivi_quantize_k_varlen",
           "kivi_quantize_v_varlen",
           "kivi_append_flush_varlen", "kivi_decode_attn_varlen", "kivi_append_decode_varlen",
           "kivi_append_decode_varlen_host",
           "kivi_fp8_cache_sizes",
           "kivi_fp8_quantize", "kivi_fp8_append", "kivi_fp8_decode_workspace_bytes",
           "kivi_fp8_decode_attn",
           "kivi_mxfp4_cache_sizes", "kivi_mxfp4_quantize", "kivi_mxfp4_append",
           "kivi_mxfp4_decode_workspace_bytes", "kivi_mxfp4_decode_attn",
           "kivi_mxfp4_append_decode",
           "kivi_decode_workspace_bytes_split", "kivi_decode_splits", "kivi_last_error",
           "kivi_time_next_decode", "kivi_abi_version")


class KiviError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class kivi_dims(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_k", ctypes.c_int32), ("group_v", ctypes.c_int32),
                ("residual", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("aging", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64)]


AGING = {"window": 0, "group": 1}    # KIVI_AGING_WINDOW, KIVI_AGING_GROUP
FLAG_VALUE_TOKEN_WINDOW = 1          # KIVI_FLAG_VALUE_TOKEN_WINDOW
FLAG_DETERMINISTIC = 2               # KIVI_FLAG_DETERMINISTIC
BUFFERS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid",
           "scale_max")


class kivi_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS]


class kivi_paging(ctypes.Structure):
    _fields_ = [("page_tokens", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
                ("pages", ctypes.c_int64), ("block_table", ctypes.c_void_p)]


class kivi_fp8_dims(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("format", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64)]


FP8_BUFFERS = ("k", "v", "k_scale", "v_scale")
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


class kivi_fp8_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in FP8_BUFFERS]


class kivi_mxfp4_dims(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64)]


MX_BUFFERS = ("k", "k_scale", "v", "v_scale")


class kivi_mxfp4_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MX_BUFFERS]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with `python bit_quantization_amd/build.py` "
                          f"(the HIP path has no fallback)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    D, C = ctypes.POINTER(kivi_dims), ctypes.POINTER(kivi_cache)
    PG = ctypes.POINTER(kivi_paging)
    MD, MC = ctypes.POINTER(kivi_mxfp4_dims), ctypes.POINTER(kivi_mxfp4_cache)
    sig = {
        "kivi_cache_sizes": (I32, [D, ctypes.POINTER(SZ)]),
        "kivi_quantize_k": (I32, [D, C, I32, P, I64, I64, P]),
        "kivi_quantize_v": (I32, [D, C, I32, P, I64, I64, P]),
        "kivi_append_flush": (I32, [D, C, I32, I64, P, P, P]),
        "kivi_decode_workspace_bytes": (I32, [D, I64, ctypes.POINTER(SZ)]),
        "kivi_decode_workspace_bytes_split": (I32, [D, I64, I32, ctypes.POINTER(SZ)]),
        "kivi_decode_splits": (I32, [D, I64, ctypes.POINTER(I32)]),
        "kivi_decode_attn": (I32, [D, C, I32, I64, P, F32, P, P, SZ, P]),
        "kivi_decode_attn_split": (I32, [D, C, I32, I64, P, F32, P, P, SZ, I32, P]),
        "kivi_append_decode": (I32, [D, C, I32, I64, P, P, P, F32, P, P, SZ, P]),
        "kivi_append_decode_noalloc": (I32, [D, C, I32, I64, P, P, P, F32, P, P]),
        "kivi_paged_cache_sizes": (I32, [D, PG, ctypes.POINTER(SZ)]),
        "kivi_quantize_k_varlen": (I32, [D, C, PG, I32, P, P, I64, I64, P]),
        "kivi_quantize_v_varlen": (I32, [D, C, PG, I32, P, P, I64, I64, P]),
        "kivi_append_flush_varlen": (I32, [D, C, PG, I32, P, I64, P, P, P]),
        "kivi_decode_attn_varlen": (I32, [D, C, PG, I32, P, I64, P, F32, P, P, SZ, P]),
        "kivi_append_decode_varlen": (I32, [D, C, PG, I32, P, I64, P, P, P, F32, P, P, SZ, P]),
        "kivi_append_decode_varlen_host": (I32, [D, C, PG, I32, P, P, I64, P, P, P, F32, P, P,
                                                 SZ, P]),
        "kivi_fp8_cache_sizes": (I32, [ctypes.POINTER(kivi_fp8_dims), ctypes.POINTER(SZ)]),
        "kivi_fp8_quantize": (I32, [ctypes.POINTER(kivi_fp8_dims), ctypes.POINTER(kivi_fp8_cache),
                                    I32, P, P, I64, I64, P]),
        "kivi_fp8_append": (I32, [ctypes.POINTER(kivi_fp8_dims), ctypes.POINTER(kivi_fp8_cache),
                                  I32, I64, P, P, P]),
        "kivi_fp8_decode_workspace_bytes": (I32, [ctypes.POINTER(kivi_fp8_dims), I64, I32,
                                                  ctypes.POINTER(SZ)]),
        "kivi_fp8_decode_attn": (I32, [ctypes.POINTER(kivi_fp8_dims),
                                       ctypes.POINTER(kivi_fp8_cache), I32, I64, P, F32, P, P,
                                       SZ, I32, P]),
        "kivi_mxfp4_cache_sizes": (I32, [MD, ctypes.POINTER(SZ)]),
        "kivi_mxfp4_quantize": (I32, [MD, MC, I32, P, P, I64, I64, P]),
        "kivi_mxfp4_append": (I32, [MD, MC, I32, I64, P, P, P]),
        "kivi_mxfp4_decode_workspace_bytes": (I32, [MD, I64, I32, ctypes.POINTER(SZ)]),
        "kivi_mxfp4_decode_attn": (I32, [MD, MC, I32, I64, P, F32, P, P, SZ, I32, P]),
        "kivi_mxfp4_append_decode": (I32, [MD, MC, I32, I64, P, P, P, F32, P, P, SZ, P]),
        "kivi_last_error": (ctypes.c_char_p, []),
        "kivi_time_next_decode": (I32, [P, P]),
        "kivi_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def _check(status: int):
    if status != 0:
        raise KiviError(status, _lib.kivi_last_error().decode())


def _ptr(t, dtype, name, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library works on device memory)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Dims:
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    bits: int
    group_k: int
    group_v: int
    residual: int
    max_tokens: int
    sink: int = 0        # tokens kept in float16 at the start of every sequence
    aging: str = "window"  # "window": a full window flushes whole; "group": its oldest group
    v_window: str = "flush"  # "flush": Values leave with the Keys; "token": one at a time
    deterministic: bool = False  # decode output bits repeat exactly (fixed block order)

    def c(self) -> kivi_dims:
        flags = ((FLAG_VALUE_TOKEN_WINDOW if self.v_window == "token" else 0)
                 | (-1 if self.v_window not in ("flush", "token") else 0)
                 | (FLAG_DETERMINISTIC if self.deterministic else 0))
        return kivi_dims(self.layers, self.batch, self.kv_heads, self.q_heads, self.head_dim,
                         self.bits, self.group_k, self.group_v, self.residual, self.sink,
                         AGING.get(self.aging, -1), flags, self.max_tokens)


def kivi_cache_sizes(dims: Dims):
    out = (ctypes.c_size_t * len(BUFFERS))()
    _check(_lib.kivi_cache_sizes(ctypes.byref(dims.c()), out))
    return list(out)


class Cache:
    """The nine caller-owned device buffers of a cache, allocated with torch."""

    def __init__(self, dims: Dims, device="cuda"):
        self.dims = dims
        sizes = kivi_cache_sizes(dims)
        self.buffers = {}
        for name, nbytes in zip(BUFFERS, sizes):
            self.buffers[name] = torch.zeros(nbytes, dtype=torch.uint8, device=device)

    def c(self) -> kivi_cache:
        return kivi_cache(*[self.buffers[n].data_ptr() for n in BUFFERS])

    # typed views (for reading results back)
    def view(self, name: str):
        d = self.dims
        L, B, H, T, D = d.layers, d.batch, d.kv_heads, d.max_tokens, d.head_dim
        buf = self.buffers[name]
        if name == "k_codes":
            return buf.view(L, B, H, T, D * d.bits // 8)
        if name in ("k_scale", "k_zero"):
            return buf.view(torch.float16).view(L, B, H, T // d.group_k, D)
        if name == "v_codes":
            return buf.view(L, B, H, T // 16, D, 16 * d.bits // 8)
        if name in ("v_scale", "v_zero"):
            return buf.view(torch.float16).view(L, B, H, T, D // d.group_v)
        if name in ("k_resid", "v_resid"):
            return buf.view(torch.float16).view(L, B, H, d.sink + d.residual, D)
        if name == "scale_max":
            return buf.view(torch.float32).view(L, B, H, 2)
        raise KeyError(name)


@dataclass
class Paging:
    """A paged cache's page geometry and block table (device int32 [B][pages_per_seq])."""
    page_tokens: int
    pages_per_seq: int
    pages: int
    block_table: torch.Tensor | None = None

    def c(self, dims: Dims | None = None) -> kivi_paging:
        bt = None
        if self.block_table is not None:
            need = dims.batch * self.pages_per_seq if dims is not None else None
            bt = _ptr(self.block_table, torch.int32, "block_table", need)
        return kivi_paging(self.page_tokens, self.pages_per_seq, self.pages, bt)


def kivi_paged_cache_sizes(dims: Dims, paging: Paging):
    out = (ctypes.c_size_t * len(BUFFERS))()
    _check(_lib.kivi_paged_cache_sizes(ctypes.byref(dims.c()), ctypes.byref(paging.c()), out))
    return list(out)


class PagedCache(Cache):
    """The nine buffers of a paged cache: the history buffers hold per layer and KV head
    a pool of pages; the window buffers and scale_max are per (sequence, KV head)."""

    def __init__(self, dims: Dims, paging: Paging, device="cuda"):
        self.dims = dims
        self.paging = paging
        self.buffers = {name: torch.zeros(nbytes, dtype=torch.uint8, device=device)
                        for name, nbytes in zip(BUFFERS, kivi_paged_cache_sizes(dims, paging))}

    def view(self, name: str):
        d, pg = self.dims, self.paging
        L, H, N, P, D = d.layers, d.kv_heads, pg.pages, pg.page_tokens, d.head_dim
        buf = self.buffers[name]
        if name == "k_codes":
            return buf.view(L, H, N, P, D * d.bits // 8)
        if name in ("k_scale", "k_zero"):
            return buf.view(torch.float16).view(L, H, N, P // d.group_k, D)
        if name == "v_codes":
            return buf.view(L, H, N, P // 16, D, 16 * d.bits // 8)
        if name in ("v_scale", "v_zero"):
            return buf.view(torch.float16).view(L, H, N, P, D // d.group_v)
        return super().view(name)

    def sequence_view(self, name: str, layer: int, b: int):
        """History buffer `name` of sequence b in token order: the pages its block-table
        row names, concatenated ([H][pages_per_seq * rows per page][...])."""
        pages = self.paging.block_table[b].long()
        v = self.view(name)[layer][:, pages]
        return v.reshape(v.shape[0], -1, *v.shape[3:])


def kivi_quantize_k(dims: Dims, cache: Cache, layer: int, k: torch.Tensor, T: int,
                    ld_tokens: int | None = None, stream=None):
    ld = T if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T else None
    _check(_lib.kivi_quantize_k(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                _ptr(k, torch.float16, "k", need), T, ld, _stream(stream)))


def kivi_quantize_v(dims: Dims, cache: Cache, layer: int, v: torch.Tensor, T: int,
                    ld_tokens: int | None = None, stream=None):
    ld = T if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T else None
    _check(_lib.kivi_quantize_v(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                _ptr(v, torch.float16, "v", need), T, ld, _stream(stream)))


def kivi_append_flush(dims: Dims, cache: Cache, layer: int, T_before: int, k_new, v_new,
                      stream=None):
    need = dims.batch * dims.kv_heads * dims.head_dim
    _check(_lib.kivi_append_flush(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                  T_before, _ptr(k_new, torch.float16, "k_new", need),
                                  _ptr(v_new, torch.float16, "v_new", need), _stream(stream)))


def kivi_decode_workspace_bytes(dims: Dims, T: int, n_split: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kivi_decode_workspace_bytes_split(ctypes.byref(dims.c()), T, n_split,
                                                  ctypes.byref(n)))
    return n.value


def kivi_decode_splits(dims: Dims, T: int) -> int:
    n = ctypes.c_int32()
    _check(_lib.kivi_decode_splits(ctypes.byref(dims.c()), T, ctypes.byref(n)))
    return n.value


def new_workspace(dims: Dims, T: int, n_split: int = 0, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (the contract asks for zeros before first use)."""
    return torch.zeros(kivi_decode_workspace_bytes(dims, T, n_split), dtype=torch.uint8,
                       device=device)


def kivi_decode_attn(dims: Dims, cache: Cache, layer: int, T: int, q: torch.Tensor,
                     sm_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                     n_split: int = 0, stream=None):
    nq = dims.batch * dims.q_heads * dims.head_dim
    qp = _ptr(q, torch.float16, "q", nq)
    op = _ptr(out, torch.float32, "out", nq)
    wp = _ptr(workspace, torch.uint8, "workspace")
    wb = workspace.numel()
    if n_split:
        st = _lib.kivi_decode_attn_split(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                         T, qp, ctypes.c_float(sm_scale), op, wp, wb, n_split,
                                         _stream(stream))
    else:
        st = _lib.kivi_decode_attn(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer, T,
                                   qp, ctypes.c_float(sm_scale), op, wp, wb, _stream(stream))
    _check(st)


def kivi_append_decode(dims: Dims, cache: Cache, layer: int, T_before: int, k_new, v_new,
                       q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                       workspace: torch.Tensor, stream=None):
    need = dims.batch * dims.kv_heads * dims.head_dim
    nq = dims.batch * dims.q_heads * dims.head_dim
    _check(_lib.kivi_append_decode(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                   T_before, _ptr(k_new, torch.float16, "k_new", need),
                                   _ptr(v_new, torch.float16, "v_new", need),
                                   _ptr(q, torch.float16, "q", nq), ctypes.c_float(sm_scale),
                                   _ptr(out, torch.float32, "out", nq),
                                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                   _stream(stream)))


# ---- ragged batches: per-sequence token counts in a device int32 [B] tensor ----------

def _lens(lens, dims):
    return _ptr(lens, torch.int32, "lens", dims.batch)


def _host_lens(lens, dims):
    """A host int32 [B] tensor's address (the library reads it during each call)."""
    if not isinstance(lens, torch.Tensor):
        raise TypeError("T_before_host must be a torch.Tensor")
    if lens.is_cuda or lens.dtype != torch.int32 or not lens.is_contiguous():
        raise ValueError("T_before_host must be a contiguous int32 CPU tensor")
    if lens.numel() < dims.batch:
        raise ValueError(f"T_before_host has {lens.numel()} elements, needs {dims.batch}")
    return lens.data_ptr()


def _paging(paging, dims):
    return None if paging is None else ctypes.byref(paging.c(dims))


def kivi_quantize_k_varlen(dims: Dims, cache: Cache, layer: int, k: torch.Tensor,
                           lens: torch.Tensor, T_hi: int, ld_tokens: int | None = None,
                           stream=None, paging: Paging | None = None):
    ld = T_hi if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T_hi else None
    _check(_lib.kivi_quantize_k_varlen(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                       _paging(paging, dims), layer,
                                       _ptr(k, torch.float16, "k", need), _lens(lens, dims),
                                       T_hi, ld, _stream(stream)))


def kivi_quantize_v_varlen(dims: Dims, cache: Cache, layer: int, v: torch.Tensor,
                           lens: torch.Tensor, T_hi: int, ld_tokens: int | None = None,
                           stream=None, paging: Paging | None = None):
    ld = T_hi if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T_hi else None
    _check(_lib.kivi_quantize_v_varlen(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                       _paging(paging, dims), layer,
                                       _ptr(v, torch.float16, "v", need), _lens(lens, dims),
                                       T_hi, ld, _stream(stream)))


def kivi_append_flush_varlen(dims: Dims, cache: Cache, layer: int, T_before: torch.Tensor,
                             T_hi: int, k_new, v_new, stream=None, paging: Paging | None = None):
    need = dims.batch * dims.kv_heads * dims.head_dim
    _check(_lib.kivi_append_flush_varlen(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                         _paging(paging, dims), layer,
                                         _lens(T_before, dims), T_hi,
                                         _ptr(k_new, torch.float16, "k_new", need),
                                         _ptr(v_new, torch.float16, "v_new", need),
                                         _stream(stream)))


def kivi_decode_attn_varlen(dims: Dims, cache: Cache, layer: int, lens: torch.Tensor, T_hi: int,
                            q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                            workspace: torch.Tensor, stream=None, paging: Paging | None = None):
    nq = dims.batch * dims.q_heads * dims.head_dim
    _check(_lib.kivi_decode_attn_varlen(ctypes.byref(dims.c()), ctypes.byref(cache.c()),
                                        _paging(paging, dims), layer,
                                        _lens(lens, dims), T_hi, _ptr(q, torch.float16, "q", nq),
                                        ctypes.c_float(sm_scale),
                                        _ptr(out, torch.float32, "out", nq),
                                        _ptr(workspace, torch.uint8, "workspace"),
                                        workspace.numel(), _stream(stream)))


def prepare_append_decode_varlen(dims: Dims, cache: Cache, layer: int, T_before: torch.Tensor,
                                 T_hi: int, k_new, v_new, q: torch.Tensor, sm_scale: float,
                                 out: torch.Tensor, workspace: torch.Tensor, stream=None,
                                 paging: Paging | None = None,
                                 T_before_host: torch.Tensor | None = None):
    """kivi_append_decode_varlen with its arguments marshalled once (see
    prepare_append_decode).  With T_before_host (a CPU int32 copy of T_before, read at
    each call, so the caller may update it in place) the call is
    kivi_append_decode_varlen_host, which skips the flush launch on steps without one."""
    need = dims.batch * dims.kv_heads * dims.head_dim
    nq = dims.batch * dims.q_heads * dims.head_dim
    pg = None if paging is None else paging.c(dims)    # kept alive by the closure
    head = (ctypes.byref(dims.c()), ctypes.byref(cache.c()),
            None if pg is None else ctypes.byref(pg), layer, _lens(T_before, dims))
    tail = (T_hi, _ptr(k_new, torch.float16, "k_new", need),
            _ptr(v_new, torch.float16, "v_new", need), _ptr(q, torch.float16, "q", nq),
            ctypes.c_float(sm_scale), _ptr(out, torch.float32, "out", nq),
            _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    if T_before_host is None:
        args = head + tail
        fn = _lib.kivi_append_decode_varlen
    else:
        args = head + (_host_lens(T_before_host, dims),) + tail
        fn = _lib.kivi_append_decode_varlen_host

    def call():
        _check(fn(*args))
    return call


def kivi_append_decode_noalloc(dims: Dims, cache: Cache, layer: int, T_before: int, k_new,
                               v_new, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                               stream=None):
    """kivi_append_decode without a workspace (the library's static decode scratch)."""
    need = dims.batch * dims.kv_heads * dims.head_dim
    nq = dims.batch * dims.q_heads * dims.head_dim
    _check(_lib.kivi_append_decode_noalloc(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                           T_before, _ptr(k_new, torch.float16, "k_new", need),
                                           _ptr(v_new, torch.float16, "v_new", need),
                                           _ptr(q, torch.float16, "q", nq),
                                           ctypes.c_float(sm_scale),
                                           _ptr(out, torch.float32, "out", nq), _stream(stream)))


def kivi_append_decode_varlen(dims: Dims, cache: Cache, layer: int, T_before: torch.Tensor,
                              T_hi: int, k_new, v_new, q: torch.Tensor, sm_scale: float,
                              out: torch.Tensor, workspace: torch.Tensor, stream=None,
                              paging: Paging | None = None,
                              T_before_host: torch.Tensor | None = None):
    prepare_append_decode_varlen(dims, cache, layer, T_before, T_hi, k_new, v_new, q, sm_scale,
                                 out, workspace, stream, paging, T_before_host)()


def prepare_append_decode(dims: Dims, cache: Cache, layer: int, T_before: int, k_new, v_new,
                          q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                          workspace: torch.Tensor, stream=None):
    """kivi_append_decode with its arguments checked and marshalled once: returns a
    function of no arguments that makes the call (for loops where the host's per-call
    cost matters; the tensors must stay alive and in place until then)."""
    need = dims.batch * dims.kv_heads * dims.head_dim
    nq = dims.batch * dims.q_heads * dims.head_dim
    args = (ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer, T_before,
            _ptr(k_new, torch.float16, "k_new", need), _ptr(v_new, torch.float16, "v_new", need),
            _ptr(q, torch.float16, "q", nq), ctypes.c_float(sm_scale),
            _ptr(out, torch.float32, "out", nq), _ptr(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream(stream))
    fn = _lib.kivi_append_decode

    def call():
        st = fn(*args)
        if st != 0:
            _check(st)
    return call


# ---- FP8 KV cache ----------------------------------------------------------------------

@dataclass
class Fp8Dims:
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    format: str          # "e4m3" or "e5m2"
    max_tokens: int

    def c(self) -> kivi_fp8_dims:
        return kivi_fp8_dims(self.layers, self.batch, self.kv_heads, self.q_heads, self.head_dim,
                             FP8_FORMATS[self.format], self.max_tokens)


def kivi_fp8_cache_sizes(dims: Fp8Dims):
    out = (ctypes.c_size_t * 4)()
    _check(_lib.kivi_fp8_cache_sizes(ctypes.byref(dims.c()), out))
    return list(out)


class Fp8Cache:
    """The four caller-owned device buffers of an FP8 cache (codes zero-filled); the
    scales [L][H_kv] are set from k_scale / v_scale (scalars or per-head arrays)."""

    def __init__(self, dims: Fp8Dims, k_scale=1.0, v_scale=1.0, device="cuda"):
        self.dims = dims
        sizes = kivi_fp8_cache_sizes(dims)
        self.buffers = {n: torch.zeros(sz, dtype=torch.uint8, device=device)
                        for n, sz in zip(FP8_BUFFERS, sizes)}
        shape = (dims.layers, dims.kv_heads)
        for name, val in (("k_scale", k_scale), ("v_scale", v_scale)):
            t = torch.as_tensor(val, dtype=torch.float32).expand(shape).contiguous()
            self.buffers[name].view(torch.float32).copy_(t.flatten().to(device))

    def c(self) -> kivi_fp8_cache:
        return kivi_fp8_cache(*[self.buffers[n].data_ptr() for n in FP8_BUFFERS])

    def view(self, name: str):
        d = self.dims
        L, B, H, T, D = d.layers, d.batch, d.kv_heads, d.max_tokens, d.head_dim
        if name == "k":
            return self.buffers[name].view(L, B, H, T, D)
        if name == "v":
            return self.buffers[name].view(L, B, H, T // 32, D, 32)
        return self.buffers[name].view(torch.float32).view(L, H)


def kivi_fp8_quantize(dims: Fp8Dims, cache: Fp8Cache, layer: int, k: torch.Tensor,
                      v: torch.Tensor, T: int, ld_tokens: int | None = None, stream=None):
    ld = T if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T else None
    _check(_lib.kivi_fp8_quantize(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                  _ptr(k, torch.float16, "k", need),
                                  _ptr(v, torch.float16, "v", need), T, ld, _stream(stream)))


def kivi_fp8_append(dims: Fp8Dims, cache: Fp8Cache, layer: int, T_before: int, k_new, v_new,
                    stream=None):
    need = dims.batch * dims.kv_heads * dims.head_dim
    _check(_lib.kivi_fp8_append(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer, T_before,
                                _ptr(k_new, torch.float16, "k_new", need),
                                _ptr(v_new, torch.float16, "v_new", need), _stream(stream)))


def kivi_fp8_decode_workspace_bytes(dims: Fp8Dims, T: int, n_split: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kivi_fp8_decode_workspace_bytes(ctypes.byref(dims.c()), T, n_split,
                                                ctypes.byref(n)))
    return n.value


def new_fp8_workspace(dims: Fp8Dims, T: int, n_split: int = 0, device="cuda") -> torch.Tensor:
    return torch.zeros(kivi_fp8_decode_workspace_bytes(dims, T, n_split), dtype=torch.uint8,
                       device=device)


def kivi_fp8_decode_attn(dims: Fp8Dims, cache: Fp8Cache, layer: int, T: int, q: torch.Tensor,
                         sm_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                         n_split: int = 0, stream=None):
    nq = dims.batch * dims.q_heads * dims.head_dim
    _check(_lib.kivi_fp8_decode_attn(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer, T,
                                     _ptr(q, torch.float16, "q", nq), ctypes.c_float(sm_scale),
                                     _ptr(out, torch.float32, "out", nq),
                                     _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                     n_split, _stream(stream)))


# ---- MXFP4 KV cache --------------------------------------------------------------------

@dataclass
class MxDims:
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    max_tokens: int

    def c(self) -> kivi_mxfp4_dims:
        return kivi_mxfp4_dims(self.layers, self.batch, self.kv_heads, self.q_heads,
                               self.head_dim, 0, self.max_tokens)


def kivi_mxfp4_cache_sizes(dims: MxDims):
    out = (ctypes.c_size_t * 4)()
    _check(_lib.kivi_mxfp4_cache_sizes(ctypes.byref(dims.c()), out))
    return list(out)


class MxCache:
    """The four caller-owned device buffers of an MXFP4 cache (zero-filled)."""

    def __init__(self, dims: MxDims, device="cuda"):
        self.dims = dims
        self.buffers = {n: torch.zeros(sz, dtype=torch.uint8, device=device)
                        for n, sz in zip(MX_BUFFERS, kivi_mxfp4_cache_sizes(dims))}

    def c(self) -> kivi_mxfp4_cache:
        return kivi_mxfp4_cache(*[self.buffers[n].data_ptr() for n in MX_BUFFERS])

    def view(self, name: str):
        d = self.dims
        L, B, H, T, D = d.layers, d.batch, d.kv_heads, d.max_tokens, d.head_dim
        buf = self.buffers[name]
        if name == "k":
            return buf.view(L, B, H, T, D // 2)
        if name == "k_scale":
            return buf.view(L, B, H, T, D // 32)
        if name == "v":
            return buf.view(L, B, H, T // 32, D, 16)
        return buf.view(L, B, H, T // 32, D // 32, 32)


def kivi_mxfp4_quantize(dims: MxDims, cache: MxCache, layer: int, k: torch.Tensor,
                        v: torch.Tensor, T: int, ld_tokens: int | None = None, stream=None):
    ld = T if ld_tokens is None else ld_tokens
    need = dims.batch * dims.kv_heads * ld * dims.head_dim if T else None
    _check(_lib.kivi_mxfp4_quantize(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                    _ptr(k, torch.float16, "k", need),
                                    _ptr(v, torch.float16, "v", need), T, ld, _stream(stream)))


def kivi_mxfp4_append(dims: MxDims, cache: MxCache, layer: int, T_before: int, k_new, v_new,
                      stream=None):
    need = dims.batch * dims.kv_heads * dims.head_dim
    _check(_lib.kivi_mxfp4_append(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                  T_before, _ptr(k_new, torch.float16, "k_new", need),
                                  _ptr(v_new, torch.float16, "v_new", need), _stream(stream)))


def kivi_mxfp4_decode_workspace_bytes(dims: MxDims, T: int, n_split: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kivi_mxfp4_decode_workspace_bytes(ctypes.byref(dims.c()), T, n_split,
                                                  ctypes.byref(n)))
    return n.value


def new_mxfp4_workspace(dims: MxDims, T: int, n_split: int = 0, device="cuda") -> torch.Tensor:
    return torch.zeros(kivi_mxfp4_decode_workspace_bytes(dims, T, n_split), dtype=torch.uint8,
                       device=device)


def kivi_mxfp4_decode_attn(dims: MxDims, cache: MxCache, layer: int, T: int, q: torch.Tensor,
                           sm_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                           n_split: int = 0, stream=None):
    nq = dims.batch * dims.q_heads * dims.head_dim
    _check(_lib.kivi_mxfp4_decode_attn(ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer,
                                       T, _ptr(q, torch.float16, "q", nq), ctypes.c_float(sm_scale),
                                       _ptr(out, torch.float32, "out", nq),
                                       _ptr(workspace, torch.uint8, "workspace"),
                                       workspace.numel(), n_split, _stream(stream)))


def prepare_mxfp4_step(dims: MxDims, cache: MxCache, layer: int, T_before: int, k_new, v_new,
                       q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                       workspace: torch.Tensor, stream=None):
    """kivi_mxfp4_append_decode (one decode step, one launch) with its arguments
    marshalled once; returns a function of no arguments making the call."""
    need = dims.batch * dims.kv_heads * dims.head_dim
    nq = dims.batch * dims.q_heads * dims.head_dim
    args = (ctypes.byref(dims.c()), ctypes.byref(cache.c()), layer, T_before,
            _ptr(k_new, torch.float16, "k_new", need), _ptr(v_new, torch.float16, "v_new", need),
            _ptr(q, torch.float16, "q", nq), ctypes.c_float(sm_scale),
            _ptr(out, torch.float32, "out", nq), _ptr(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream(stream))
    fn = _lib.kivi_mxfp4_append_decode

    def call():
        _check(fn(*args))
    return call


def kivi_mxfp4_append_decode(dims: MxDims, cache: MxCache, layer: int, T_before: int, k_new,
                             v_new, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                             workspace: torch.Tensor, stream=None):
    prepare_mxfp4_step(dims, cache, layer, T_before, k_new, v_new, q, sm_scale, out, workspace,
                       stream)()


def kivi_time_next_decode(start=None, stop=None):
    """Arm the calling thread's next decode-kernel launch to record two events (raw
    hipEvent_t handles as ints, e.g. torch.cuda.Event(enable_timing=True).cuda_event
    after a first record) at the kernel's own start and end; no arguments disarm."""
    _check(_lib.kivi_time_next_decode(start, stop))


def kivi_abi_version() -> int:
    return int(_lib.kivi_abi_version())
