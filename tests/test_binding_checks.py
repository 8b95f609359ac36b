"""The Python binding refuses buffers too small for the call before the
library sees their plain pointers (CPU: no library call is made)."""
from __future__ import annotations

import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp

L, W = 512, 32


def _meta():
    return ibp.Meta(None, L, W)  # no handle: every call below must stop before the library


def _bytes(n):
    return torch.zeros(n, dtype=torch.uint8)


@pytest.mark.parametrize("which", ["src", "dst_slots", "bitmask", "stored_bytes"])
def test_compress_short_buffers(which):
    n = 40
    args = dict(src=_bytes(n * L), dst_slots=_bytes(n * L), bitmask=torch.zeros(2, dtype=torch.int32),
                stored_bytes=torch.zeros(n, dtype=torch.int64))
    short = {"src": _bytes(n * L - 1), "dst_slots": _bytes(n * L - 16), "bitmask": torch.zeros(1, dtype=torch.int32),
             "stored_bytes": torch.zeros(n - 1, dtype=torch.int64)}
    args[which] = short[which]
    with pytest.raises(ValueError, match=which):
        ibp.ibp_compress(_meta(), args["src"], n, args["dst_slots"], args["bitmask"], args["stored_bytes"])


def test_decode_short_buffers():
    n = 64
    m = _meta()
    with pytest.raises(ValueError, match="dst"):
        ibp.ibp_decompress(m, _bytes(n * L), torch.zeros(2, dtype=torch.int32), n, _bytes(n * L - 4))
    with pytest.raises(ValueError, match="slots"):
        ibp.ibp_decompress(m, _bytes(L), torch.zeros(2, dtype=torch.int32), n, _bytes(n * L))
    ids = torch.zeros(10, dtype=torch.int64)
    with pytest.raises(ValueError, match="dst"):
        ibp.ibp_gather_decompress(m, _bytes(n * L), n, torch.zeros(2, dtype=torch.int32), ids, _bytes(9 * L))
    with pytest.raises(ValueError, match="bitmask"):
        ibp.ibp_gather_decompress(m, _bytes(n * L), n, torch.zeros(1, dtype=torch.int32), ids, _bytes(10 * L))


def test_packed_and_split_short_buffers():
    n = 33
    m = _meta()
    off = torch.zeros(n + 1, dtype=torch.int64)
    bm = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="capacity"):
        ibp.ibp_compress_packed(m, _bytes(n * L), n, off, _bytes(100), bm, capacity=101)
    with pytest.raises(ValueError, match="buf_bytes"):
        ibp.ibp_decompress_packed(m, _bytes(100), off, bm, n, _bytes(n * L), buf_bytes=200)
    with pytest.raises(ValueError, match="offsets"):
        ibp.ibp_gather_decompress_packed(m, _bytes(100), off[:n], n, bm, torch.zeros(1, dtype=torch.int64),
                                         _bytes(L))
    with pytest.raises(ValueError, match="headers"):
        ibp.ibp_compress_split(m, _bytes(n * L), n, _bytes(n * L), torch.zeros(n - 1, dtype=torch.int32), bm)
    with pytest.raises(ValueError, match="headers"):
        ibp.ibp_gather_decompress_split(m, _bytes(n * L), n, torch.zeros(1, dtype=torch.int32), bm,
                                        torch.zeros(1, dtype=torch.int64), _bytes(L))
