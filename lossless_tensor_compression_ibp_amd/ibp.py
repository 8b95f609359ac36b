"""Python binding of libibp (include/ibp.h): argument marshalling only.

Every function forwards torch tensors (device memory, or pinned host memory
where the C ABI allows it) as raw pointers together with the HIP stream of
torch's current stream.  All codec work runs in the gfx950 kernels of
libibp.so; if the library is missing this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libibp.so")

IBP_OK = 0
IBP_ERR_INVALID_ARG = -1
IBP_ERR_UNSUPPORTED = -2
IBP_ERR_DEVICE = -3
IBP_ERR_NOMEM = -4
IBP_ERR_CORRUPT = -5
IBP_ERR_RANGE = -6
IBP_ERR_TOO_LARGE = -7

# ibp_decompress_noalloc's static scratch (include/ibp.h)
NOALLOC_SCRATCH_BYTES = 1 << 20
NOALLOC_MAX_TILES = NOALLOC_SCRATCH_BYTES // 8 - 32

# every function the header declares (checked by the tests)
ABI_FUNCTIONS = (
    "ibp_build_metadata", "ibp_meta_create", "ibp_meta_get", "ibp_meta_get_info",
    "ibp_meta_set_first_read", "ibp_meta_destroy", "ibp_compress", "ibp_decompress", "ibp_gather_decompress",
    "ibp_check", "ibp_status_string",
    "ibp_packed_offsets", "ibp_compress_packed", "ibp_decompress_packed", "ibp_gather_decompress_packed",
    "ibp_compress_split", "ibp_decompress_split", "ibp_gather_decompress_split",
    "ibp_decompress_noalloc",
)


class ibp_params(ctypes.Structure):
    _fields_ = [("tensor_bytes", ctypes.c_uint64), ("chunk_bits", ctypes.c_uint32),
                ("period_bits", ctypes.c_uint32), ("threshold", ctypes.c_double)]


class ibp_meta_info(ctypes.Structure):
    _fields_ = [("invariant_bits", ctypes.c_uint64), ("min_record_bytes", ctypes.c_uint64),
                ("max_runs", ctypes.c_uint32), ("uniform", ctypes.c_uint32)]


class IBPError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """Load libibp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m lossless_tensor_compression_ibp_amd.build_lib")
        L = ctypes.CDLL(LIB_PATH)
        p, u64, st = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
        P = ctypes.POINTER
        L.ibp_build_metadata.argtypes = [P(ibp_params), p, u64, P(p), p]
        L.ibp_meta_create.argtypes = [P(ibp_params), p, p, P(p), p]
        L.ibp_meta_get.argtypes = [p, P(ibp_params), p, p]
        L.ibp_meta_get_info.argtypes = [p, P(ibp_meta_info)]
        L.ibp_meta_set_first_read.argtypes = [p, u64]
        L.ibp_meta_destroy.argtypes = [p]
        L.ibp_compress.argtypes = [p, p, u64, p, p, p, p]
        L.ibp_decompress.argtypes = [p, p, p, u64, p, p]
        L.ibp_decompress_noalloc.argtypes = [p, p, p, u64, p, p]
        L.ibp_gather_decompress.argtypes = [p, p, u64, p, p, u64, p, p]
        L.ibp_check.argtypes = [p, p]
        L.ibp_packed_offsets.argtypes = [p, p, u64, p, p]
        L.ibp_compress_packed.argtypes = [p, p, u64, p, p, u64, p, p]
        L.ibp_decompress_packed.argtypes = [p, p, u64, p, p, u64, p, p]
        L.ibp_gather_decompress_packed.argtypes = [p, p, u64, p, u64, p, p, u64, p, p]
        L.ibp_compress_split.argtypes = [p, p, u64, p, p, p, p, p]
        L.ibp_decompress_split.argtypes = [p, p, p, p, u64, p, p]
        L.ibp_gather_decompress_split.argtypes = [p, p, u64, p, p, p, u64, p, p]
        L.ibp_status_string.argtypes = [st]
        L.ibp_status_string.restype = ctypes.c_char_p
        for f in ABI_FUNCTIONS:
            if f != "ibp_status_string":
                getattr(L, f).restype = st
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ibp_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != IBP_OK:
        raise IBPError(status, what)


def _need(t: torch.Tensor | None, nbytes: int, what: str):
    """Buffers reach the library as plain pointers: check here that each one
    holds what the call will read or write."""
    if t is not None and t.nbytes < nbytes:
        raise ValueError(f"{what} holds {t.nbytes} bytes, the call needs {nbytes}")


def _bitmask_bytes(n: int) -> int:
    return 4 * ((int(n) + 31) // 32)


def _need_all(*checks):
    """(tensor, bytes, name) triples; raises for the first buffer that is too
    small.  Called only after a combined test failed, so the common path of a
    hot call costs one comparison per buffer."""
    for t, nbytes, what in checks:
        _need(t, nbytes, what)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libibp must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> ctypes.c_void_p:
    """HIP stream handle: the given torch stream, else torch's current stream
    on the current device (read without building a Stream object)."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Meta:
    """Owns an ibp_meta_t handle; keeps the tensor length L and chunk width W
    so that the calls below can check buffer sizes before the library sees
    plain pointers."""

    def __init__(self, handle: ctypes.c_void_p, tensor_bytes: int = 0, chunk_bits: int = 0):
        self.handle = handle
        self.tensor_bytes = int(tensor_bytes)
        self.chunk_bits = int(chunk_bits)
        self.hdr_words = (8 * self.tensor_bytes // self.chunk_bits + 31) // 32 if self.chunk_bits else 0

    @property
    def _as_parameter_(self):
        return self.handle

    def close(self):
        if self.handle:
            _check(lib().ibp_meta_destroy(self.handle), "ibp_meta_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _params(tensor_bytes, chunk_bits, period_bits, threshold=0.0):
    return ibp_params(int(tensor_bytes), int(chunk_bits), int(period_bits), float(threshold))


def ibp_build_metadata(sample: torch.Tensor, n_sample: int, tensor_bytes: int, chunk_bits: int,
                       period_bits: int, threshold: float, stream=None) -> Meta:
    prm = _params(tensor_bytes, chunk_bits, period_bits, threshold)
    out = ctypes.c_void_p()
    _need(sample, int(n_sample) * int(tensor_bytes), "sample")
    _check(lib().ibp_build_metadata(ctypes.byref(prm), _ptr(sample), int(n_sample), ctypes.byref(out),
                                    _stream(stream)), "ibp_build_metadata")
    return Meta(out, tensor_bytes, chunk_bits)


def ibp_meta_create(tensor_bytes: int, chunk_bits: int, period_bits: int, mask, bitval, stream=None) -> Meta:
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    bitval = np.ascontiguousarray(bitval, dtype=np.uint32)
    prm = _params(tensor_bytes, chunk_bits, period_bits)
    out = ctypes.c_void_p()
    if mask.size < period_bits // 32 or bitval.size < period_bits // 32:
        raise ValueError("mask and bitval need period_bits / 32 words each")
    _check(lib().ibp_meta_create(ctypes.byref(prm), ctypes.c_void_p(mask.ctypes.data),
                                 ctypes.c_void_p(bitval.ctypes.data), ctypes.byref(out), _stream(stream)),
           "ibp_meta_create")
    return Meta(out, tensor_bytes, chunk_bits)


def ibp_meta_get(meta: Meta):
    prm = ibp_params()
    _check(lib().ibp_meta_get(meta, ctypes.byref(prm), None, None), "ibp_meta_get")
    mw = prm.period_bits // 32
    mask = np.zeros(mw, np.uint32)
    bitval = np.zeros(mw, np.uint32)
    _check(lib().ibp_meta_get(meta, None, ctypes.c_void_p(mask.ctypes.data),
                              ctypes.c_void_p(bitval.ctypes.data)), "ibp_meta_get")
    params = dict(tensor_bytes=prm.tensor_bytes, chunk_bits=prm.chunk_bits,
                  period_bits=prm.period_bits, threshold=prm.threshold)
    return params, mask, bitval


def ibp_meta_get_info(meta: Meta) -> dict:
    info = ibp_meta_info()
    _check(lib().ibp_meta_get_info(meta, ctypes.byref(info)), "ibp_meta_get_info")
    return dict(invariant_bits=info.invariant_bits, min_record_bytes=info.min_record_bytes,
                max_runs=info.max_runs, uniform=info.uniform)


def ibp_meta_set_first_read(meta: Meta, nbytes: int):
    _check(lib().ibp_meta_set_first_read(meta, int(nbytes)), "ibp_meta_set_first_read")


def ibp_meta_destroy(meta: Meta):
    meta.close()


def ibp_compress(meta: Meta, src: torch.Tensor, n_tensors: int, dst_slots: torch.Tensor,
                 bitmask: torch.Tensor, stored_bytes: torch.Tensor | None = None, stream=None):
    L, n = meta.tensor_bytes, int(n_tensors)
    _need(src, n * L, "src")
    _need(dst_slots, n * L, "dst_slots")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(stored_bytes, 8 * n, "stored_bytes")
    _check(lib().ibp_compress(meta, _ptr(src), int(n_tensors), _ptr(dst_slots), _ptr(bitmask),
                              _ptr(stored_bytes), _stream(stream)), "ibp_compress")


def ibp_decompress(meta: Meta, slots: torch.Tensor, bitmask: torch.Tensor, n_tensors: int,
                   dst: torch.Tensor, stream=None):
    L, n = meta.tensor_bytes, int(n_tensors)
    _need(slots, n * L, "slots")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(dst, n * L, "dst")
    _check(lib().ibp_decompress(meta, _ptr(slots), _ptr(bitmask), int(n_tensors), _ptr(dst),
                                _stream(stream)), "ibp_decompress")


def ibp_decompress_noalloc(meta: Meta, slots: torch.Tensor, bitmask: torch.Tensor, n_tensors: int,
                           dst: torch.Tensor, stream=None):
    """ibp_decompress without device allocation (the library's static
    scratch); the same output."""
    L, n = meta.tensor_bytes, int(n_tensors)
    _need(slots, n * L, "slots")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(dst, n * L, "dst")
    _check(lib().ibp_decompress_noalloc(meta, _ptr(slots), _ptr(bitmask), int(n_tensors), _ptr(dst),
                                        _stream(stream)), "ibp_decompress_noalloc")


def ibp_gather_decompress(meta: Meta, slots: torch.Tensor, n_slots: int, bitmask: torch.Tensor,
                          ids: torch.Tensor, dst: torch.Tensor, stream=None):
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    L, n, k = meta.tensor_bytes, int(n_slots), ids.numel()
    if slots.nbytes < n * L or bitmask.nbytes < 4 * ((n + 31) // 32) or dst.nbytes < k * L:
        _need_all((slots, n * L, "slots"), (bitmask, _bitmask_bytes(n), "bitmask"), (dst, k * L, "dst"))
    _check(lib().ibp_gather_decompress(meta, _ptr(slots), int(n_slots), _ptr(bitmask), _ptr(ids),
                                       int(ids.numel()), _ptr(dst), _stream(stream)),
           "ibp_gather_decompress")


def ibp_check(meta: Meta, stream=None) -> int:
    """Synchronises the stream; returns the latched device status (0 = ok)."""
    return int(lib().ibp_check(meta, _stream(stream)))


# ---------------------------------------------------------------------------
# Packed cache: items back to back at 16-byte aligned offsets.
# ---------------------------------------------------------------------------
def ibp_packed_offsets(meta: Meta, src: torch.Tensor, n_tensors: int, offsets: torch.Tensor, stream=None):
    """offsets: device int64 tensor of n_tensors + 1 entries (written)."""
    if offsets.dtype != torch.int64 or offsets.numel() < n_tensors + 1:
        raise ValueError("offsets must be int64 with n_tensors + 1 entries")
    if n_tensors:
        _need(src, int(n_tensors) * meta.tensor_bytes, "src")
    _check(lib().ibp_packed_offsets(meta, _ptr(src) if n_tensors else None, int(n_tensors), _ptr(offsets),
                                    _stream(stream)), "ibp_packed_offsets")


def ibp_compress_packed(meta: Meta, src: torch.Tensor, n_tensors: int, offsets: torch.Tensor, dst: torch.Tensor,
                        bitmask: torch.Tensor, capacity: int | None = None, stream=None):
    if capacity is None:
        capacity = dst.nbytes
    elif capacity > dst.nbytes:
        raise ValueError(f"capacity {capacity} exceeds dst ({dst.nbytes} bytes)")
    n = int(n_tensors)
    _need(src, n * meta.tensor_bytes, "src")
    _need(offsets, 8 * (n + 1), "offsets")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _check(lib().ibp_compress_packed(meta, _ptr(src), int(n_tensors), _ptr(offsets), _ptr(dst), int(capacity),
                                     _ptr(bitmask), _stream(stream)), "ibp_compress_packed")


def ibp_decompress_packed(meta: Meta, buf: torch.Tensor, offsets: torch.Tensor, bitmask: torch.Tensor,
                          n_items: int, dst: torch.Tensor, buf_bytes: int | None = None, stream=None):
    if buf_bytes is None:
        buf_bytes = buf.nbytes
    elif buf_bytes > buf.nbytes:
        raise ValueError(f"buf_bytes {buf_bytes} exceeds buf ({buf.nbytes} bytes)")
    n = int(n_items)
    _need(offsets, 8 * (n + 1), "offsets")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(dst, n * meta.tensor_bytes, "dst")
    _check(lib().ibp_decompress_packed(meta, _ptr(buf), int(buf_bytes), _ptr(offsets), _ptr(bitmask),
                                       int(n_items), _ptr(dst), _stream(stream)), "ibp_decompress_packed")


def ibp_gather_decompress_packed(meta: Meta, buf: torch.Tensor, offsets: torch.Tensor, n_items: int,
                                 bitmask: torch.Tensor, ids: torch.Tensor, dst: torch.Tensor,
                                 buf_bytes: int | None = None, stream=None):
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    if buf_bytes is None:
        buf_bytes = buf.nbytes
    elif buf_bytes > buf.nbytes:
        raise ValueError(f"buf_bytes {buf_bytes} exceeds buf ({buf.nbytes} bytes)")
    n, k = int(n_items), ids.numel() * meta.tensor_bytes
    if offsets.nbytes < 8 * (n + 1) or bitmask.nbytes < 4 * ((n + 31) // 32) or dst.nbytes < k:
        _need_all((offsets, 8 * (n + 1), "offsets"), (bitmask, _bitmask_bytes(n), "bitmask"), (dst, k, "dst"))
    _check(lib().ibp_gather_decompress_packed(meta, _ptr(buf), int(buf_bytes), _ptr(offsets), int(n_items),
                                              _ptr(bitmask), _ptr(ids), int(ids.numel()), _ptr(dst),
                                              _stream(stream)), "ibp_gather_decompress_packed")


# ---------------------------------------------------------------------------
# Headers in GPU memory: header words beside the bitmask, payload in the slot.
# ---------------------------------------------------------------------------
def _header_words(meta: Meta) -> int:
    return meta.hdr_words


def header_words(meta: Meta) -> int:
    prm, _, _ = ibp_meta_get(meta)
    return (8 * prm["tensor_bytes"] // prm["chunk_bits"] + 31) // 32


def ibp_compress_split(meta: Meta, src: torch.Tensor, n_tensors: int, dst_slots: torch.Tensor,
                       headers: torch.Tensor, bitmask: torch.Tensor, stored_bytes: torch.Tensor | None = None,
                       stream=None):
    L, n = meta.tensor_bytes, int(n_tensors)
    _need(src, n * L, "src")
    _need(dst_slots, n * L, "dst_slots")
    _need(headers, 4 * n * _header_words(meta), "headers")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(stored_bytes, 8 * n, "stored_bytes")
    _check(lib().ibp_compress_split(meta, _ptr(src), int(n_tensors), _ptr(dst_slots), _ptr(headers),
                                    _ptr(bitmask), _ptr(stored_bytes), _stream(stream)), "ibp_compress_split")


def ibp_decompress_split(meta: Meta, slots: torch.Tensor, headers: torch.Tensor, bitmask: torch.Tensor,
                         n_tensors: int, dst: torch.Tensor, stream=None):
    L, n = meta.tensor_bytes, int(n_tensors)
    _need(slots, n * L, "slots")
    _need(headers, 4 * n * _header_words(meta), "headers")
    _need(bitmask, _bitmask_bytes(n), "bitmask")
    _need(dst, n * L, "dst")
    _check(lib().ibp_decompress_split(meta, _ptr(slots), _ptr(headers), _ptr(bitmask), int(n_tensors), _ptr(dst),
                                      _stream(stream)), "ibp_decompress_split")


def ibp_gather_decompress_split(meta: Meta, slots: torch.Tensor, n_slots: int, headers: torch.Tensor,
                                bitmask: torch.Tensor, ids: torch.Tensor, dst: torch.Tensor, stream=None):
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    L, n, k = meta.tensor_bytes, int(n_slots), ids.numel()
    hb = 4 * n * _header_words(meta)
    if (slots.nbytes < n * L or headers.nbytes < hb or bitmask.nbytes < 4 * ((n + 31) // 32)
            or dst.nbytes < k * L):
        _need_all((slots, n * L, "slots"), (headers, hb, "headers"), (bitmask, _bitmask_bytes(n), "bitmask"),
                  (dst, k * L, "dst"))
    _check(lib().ibp_gather_decompress_split(meta, _ptr(slots), int(n_slots), _ptr(headers), _ptr(bitmask),
                                             _ptr(ids), int(ids.numel()), _ptr(dst), _stream(stream)),
           "ibp_gather_decompress_split")
