"""ctypes wrapper over the plain C oracle (libibp_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg.  The product path never imports it.

Every function takes and returns numpy arrays; the C side walks single bits
(see ibp_oracle.h for the bit conventions and the passages of the method each
function follows).  The threshold arithmetic, the match test, the bit removal
and the reinsertion all live in C; this file only marshals buffers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libibp_oracle.so")
SRC_PATH = os.path.join(_HERE, "ibp_oracle.c")

OK, ERR_INVALID, ERR_CORRUPT, ERR_RANGE = 0, -1, -5, -6


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libibp_oracle.so."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
             "-o", tmp, SRC_PATH, "-lm"],
            check=True,
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, dbl, p = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        L.ibp_ref_build_metadata.argtypes = [u64, u32, u32, dbl, p, u64, p, p]
        L.ibp_ref_encode_record.argtypes = [u64, u32, u32, p, p, p, p, u64, p]
        L.ibp_ref_max_record_bits.argtypes = [u64, u32]
        L.ibp_ref_max_record_bits.restype = u64
        L.ibp_ref_record_bits.argtypes = [u64, u32, u32, p, p, u64, p]
        L.ibp_ref_decode_record.argtypes = [u64, u32, u32, p, p, p, u64, p]
        L.ibp_ref_encode_records.argtypes = [u64, u32, u32, p, p, p, u64, u64, p, u64, p]
        L.ibp_ref_decode_records.argtypes = [u64, u32, u32, p, p, p, u64, u64, p, u64]
        L.ibp_ref_compress.argtypes = [u64, u32, u32, p, p, p, u64, p, p, p]
        L.ibp_ref_decompress.argtypes = [u64, u32, u32, p, p, p, p, u64, p]
        L.ibp_ref_gather_decompress.argtypes = [u64, u32, u32, p, p, p, u64, p, p, u64, p]
        L.ibp_ref_packed_offsets.argtypes = [u64, u32, u32, p, p, p, u64, p]
        L.ibp_ref_compress_packed.argtypes = [u64, u32, u32, p, p, p, u64, p, u64, p, p]
        L.ibp_ref_gather_decompress_packed.argtypes = [u64, u32, u32, p, p, p, p, u64, p, p, u64, p]
        L.ibp_ref_compress_split.argtypes = [u64, u32, u32, p, p, p, u64, p, p, p, p]
        L.ibp_ref_gather_decompress_split.argtypes = [u64, u32, u32, p, p, p, u64, p, p, p, u64, p]
        for name in ("ibp_ref_build_metadata", "ibp_ref_encode_record", "ibp_ref_record_bits",
                     "ibp_ref_decode_record", "ibp_ref_encode_records", "ibp_ref_decode_records",
                     "ibp_ref_compress", "ibp_ref_decompress", "ibp_ref_gather_decompress",
                     "ibp_ref_packed_offsets", "ibp_ref_compress_packed", "ibp_ref_gather_decompress_packed",
                     "ibp_ref_compress_split", "ibp_ref_gather_decompress_split"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint8).reshape(-1)


def _check(code: int, what: str):
    if code != OK:
        raise OracleError(code, what)


def nbytes_for_bits(bits: int) -> int:
    return (bits + 7) // 8


def build_metadata(sample, tensor_bits: int, W: int, M: int, T: float, n_sample: int):
    """Mask and Bitval (uint8 bit strings of M bits) from n_sample tensors."""
    s = _u8(sample)
    assert s.size * 8 >= n_sample * tensor_bits
    mask = np.zeros(nbytes_for_bits(M), np.uint8)
    bitval = np.zeros(nbytes_for_bits(M), np.uint8)
    _check(lib().ibp_ref_build_metadata(tensor_bits, W, M, float(T), _ptr(s), n_sample,
                                        _ptr(mask), _ptr(bitval)), "build_metadata")
    return mask, bitval


def max_record_bits(tensor_bits: int, W: int) -> int:
    return int(lib().ibp_ref_max_record_bits(tensor_bits, W))


def encode_record(x, tensor_bits: int, W: int, M: int, mask, bitval):
    """Record bytes (padded to 32 bits) and its exact length R in bits."""
    xb = _u8(x)
    cap = max_record_bits(tensor_bits, W)
    rec = np.zeros(cap // 8, np.uint8)
    R = ctypes.c_uint64(0)
    _check(lib().ibp_ref_encode_record(tensor_bits, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)),
                                       _ptr(xb), _ptr(rec), cap, ctypes.byref(R)), "encode_record")
    R = int(R.value)
    return rec[: 4 * ((R + 31) // 32)].copy(), R


def record_bits(rec, tensor_bits: int, W: int, M: int, mask, avail_bits=None) -> int:
    r = _u8(rec)
    if avail_bits is None:
        avail_bits = r.size * 8
    R = ctypes.c_uint64(0)
    _check(lib().ibp_ref_record_bits(tensor_bits, W, M, _ptr(_u8(mask)), _ptr(r), avail_bits,
                                     ctypes.byref(R)), "record_bits")
    return int(R.value)


def decode_record(rec, tensor_bits: int, W: int, M: int, mask, bitval, avail_bits=None):
    r = _u8(rec)
    if avail_bits is None:
        avail_bits = r.size * 8
    x = np.zeros(nbytes_for_bits(tensor_bits), np.uint8)
    _check(lib().ibp_ref_decode_record(tensor_bits, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)),
                                       _ptr(r), avail_bits, _ptr(x)), "decode_record")
    return x


def encode_records(xs: np.ndarray, tensor_bits: int, W: int, M: int, mask, bitval):
    """xs: (n, x_stride) uint8.  Returns (records (n, rec_stride) uint8, R (n,))."""
    xs = np.ascontiguousarray(xs, dtype=np.uint8)
    n, x_stride = xs.shape
    rec_stride = max_record_bits(tensor_bits, W) // 8
    recs = np.zeros((n, rec_stride), np.uint8)
    R = np.zeros(n, np.uint64)
    _check(lib().ibp_ref_encode_records(tensor_bits, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)),
                                        _ptr(xs), n, x_stride, _ptr(recs), rec_stride, _ptr(R)),
           "encode_records")
    return recs, R


def decode_records(recs: np.ndarray, tensor_bits: int, W: int, M: int, mask, bitval):
    recs = np.ascontiguousarray(recs, dtype=np.uint8)
    n, rec_stride = recs.shape
    x_stride = nbytes_for_bits(tensor_bits)
    xs = np.zeros((n, x_stride), np.uint8)
    _check(lib().ibp_ref_decode_records(tensor_bits, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)),
                                        _ptr(recs), rec_stride, n, _ptr(xs), x_stride),
           "decode_records")
    return xs


def compress(src, L: int, W: int, M: int, mask, bitval, n_tensors: int):
    """Returns (slots uint8 (n, L), bitmask uint32 (ceil(n/32),), stored uint64 (n,))."""
    s = _u8(src)
    assert s.size >= n_tensors * L
    slots = np.zeros((n_tensors, L), np.uint8)
    bitmask = np.zeros((n_tensors + 31) // 32, np.uint32)
    stored = np.zeros(n_tensors, np.uint64)
    _check(lib().ibp_ref_compress(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), n_tensors,
                                  _ptr(slots), _ptr(bitmask), _ptr(stored)), "compress")
    return slots, bitmask, stored


def decompress(slots, bitmask, L: int, W: int, M: int, mask, bitval, n_tensors: int):
    s = _u8(slots)
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    dst = np.zeros((n_tensors, L), np.uint8)
    _check(lib().ibp_ref_decompress(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), _ptr(bm),
                                    n_tensors, _ptr(dst)), "decompress")
    return dst


def gather_decompress(slots, n_slots: int, bitmask, ids, L: int, W: int, M: int, mask, bitval):
    s = _u8(slots)
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    dst = np.zeros((ids.size, L), np.uint8)
    _check(lib().ibp_ref_gather_decompress(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s),
                                           n_slots, _ptr(bm), _ptr(ids), ids.size, _ptr(dst)),
           "gather_decompress")
    return dst


def packed_offsets(src, L: int, W: int, M: int, mask, bitval, n_tensors: int):
    """Offsets (uint64, n + 1) of the items stored back to back."""
    s = _u8(src)
    assert s.size >= n_tensors * L
    off = np.zeros(n_tensors + 1, np.uint64)
    _check(lib().ibp_ref_packed_offsets(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), n_tensors,
                                        _ptr(off)), "packed_offsets")
    return off


def compress_packed(src, L: int, W: int, M: int, mask, bitval, n_tensors: int, capacity: int | None = None):
    """Returns (buf uint8 (capacity,), offsets uint64 (n + 1,), bitmask uint32)."""
    s = _u8(src)
    assert s.size >= n_tensors * L
    if capacity is None:
        capacity = n_tensors * ((L + 15) // 16 * 16)
    buf = np.zeros(max(capacity, 1), np.uint8)
    off = np.zeros(n_tensors + 1, np.uint64)
    bitmask = np.zeros((n_tensors + 31) // 32, np.uint32)
    _check(lib().ibp_ref_compress_packed(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), n_tensors,
                                         _ptr(buf), capacity, _ptr(off), _ptr(bitmask if bitmask.size else
                                                                                np.zeros(1, np.uint32))),
           "compress_packed")
    return buf[:capacity], off, bitmask


def gather_decompress_packed(buf, offsets, n_items: int, bitmask, ids, L: int, W: int, M: int, mask, bitval):
    b = _u8(buf) if np.asarray(buf).size else np.zeros(1, np.uint8)
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    if bm.size == 0:
        bm = np.zeros(1, np.uint32)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    dst = np.zeros((ids.size, L), np.uint8)
    _check(lib().ibp_ref_gather_decompress_packed(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(b),
                                                  _ptr(off), n_items, _ptr(bm), _ptr(ids), ids.size,
                                                  _ptr(dst)), "gather_decompress_packed")
    return dst


def header_words(L: int, W: int) -> int:
    return (8 * L // W + 31) // 32


def compress_split(src, L: int, W: int, M: int, mask, bitval, n_tensors: int):
    """Returns (slots (n, L) uint8, headers (n, hw) uint32, bitmask, stored)."""
    s = _u8(src)
    assert s.size >= n_tensors * L
    hw = header_words(L, W)
    slots = np.zeros((n_tensors, L), np.uint8)
    headers = np.zeros((max(n_tensors, 1), hw), np.uint32)
    bitmask = np.zeros(max(1, (n_tensors + 31) // 32), np.uint32)
    stored = np.zeros(max(n_tensors, 1), np.uint64)
    _check(lib().ibp_ref_compress_split(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), n_tensors,
                                        _ptr(slots), _ptr(headers), _ptr(bitmask), _ptr(stored)),
           "compress_split")
    return slots, headers[:n_tensors], bitmask[: (n_tensors + 31) // 32], stored[:n_tensors]


def gather_decompress_split(slots, n_slots: int, headers, bitmask, ids, L: int, W: int, M: int, mask, bitval):
    s = _u8(slots)
    h = np.ascontiguousarray(headers, dtype=np.uint32)
    bm = np.ascontiguousarray(bitmask, dtype=np.uint32)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    dst = np.zeros((ids.size, L), np.uint8)
    _check(lib().ibp_ref_gather_decompress_split(L, W, M, _ptr(_u8(mask)), _ptr(_u8(bitval)), _ptr(s), n_slots,
                                                 _ptr(h), _ptr(bm), _ptr(ids), ids.size, _ptr(dst)),
           "gather_decompress_split")
    return dst
