"""ibp_decompress_noalloc, the decode entry point for callers that cannot
allocate device memory (the start-bit scratch of its long tensors is a
static device array of the library), against ibp_decompress through the C
ABI, with the slots in device memory (header pass, scan and group decode):
the same bytes on
two calls in a row, the second with a smaller input, and inside a captured
HIP graph replayed between eager calls."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp
from lossless_tensor_compression_ibp_amd import workloads as WL
from tests.gpu_util import as_rows, device, say

pytestmark = pytest.mark.gpu


def _layers(n: int, rows: int = 40, cols: int = 1000, seed: int = 0) -> np.ndarray:
    """n bf16 tensors of rows x cols (80,000 bytes: ten 2,048-word tiles, the
    last one ragged); tensor 2 is random bytes, stored raw."""
    raw = np.stack([WL.llm_layer(l, rows=rows, cols=cols, seed=seed).reshape(-1).view(np.uint8) for l in range(n)])
    if n > 2:
        raw[2] = np.random.default_rng(seed + 7).integers(0, 256, raw.shape[1], dtype=np.uint8)
    return raw


def _encoded(raw: np.ndarray, meta=None):
    dev = device()
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    if meta is None:
        w = WL.LLM_BF16
        meta = ibp.ibp_build_metadata(src, 1, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = torch.empty_like(src)
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bm)
    torch.cuda.synchronize()
    return meta, src, slots, bm


def _both(meta, slots, bm, n, L):
    dev = device()
    ref = torch.empty((n, L), dtype=torch.uint8, device=dev)
    out = torch.full((n, L), 0xA5, dtype=torch.uint8, device=dev)
    ibp.ibp_decompress(meta, slots, bm, n, ref)
    ibp.ibp_decompress_noalloc(meta, slots, bm, n, out)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    return ref, out


def test_noalloc_matches_decompress_on_two_calls():
    raw = _layers(5)
    n, L = raw.shape
    meta, src, slots, bm = _encoded(raw)
    bits = np.unpackbits(bm.cpu().numpy().view(np.uint8), bitorder="little")[:n]
    assert bits.tolist() == [1, 1, 0, 1, 1], bits
    say(f"[noalloc] call 1: {n} tensors of {L} bytes (10 tiles each)")
    ref, out = _both(meta, slots, bm, n, L)
    assert torch.equal(out, ref) and torch.equal(out, src)
    # second call, smaller input: two other tensors (their slots), fewer tiles
    raw2 = _layers(2, seed=5)
    _, src2, slots2, bm2 = _encoded(raw2, meta)
    say("[noalloc] call 2: 2 tensors")
    ref2, out2 = _both(meta, slots2, bm2, 2, L)
    assert torch.equal(out2, ref2) and torch.equal(out2, src2)
    # single-tile tensors (no scratch): dense_gnn rows
    w = WL.DENSE_GNN
    rows = as_rows(WL.dense_gnn(2000))
    src3 = torch.from_numpy(rows).to(device())
    meta3 = ibp.ibp_build_metadata(src3, 1024, rows.shape[1], w.chunk_bits, w.period_bits, w.threshold)
    _, _, slots3, bm3 = _encoded(rows, meta3)
    for m in (2000, 777):
        say(f"[noalloc] single-tile rows: {m}")
        ref3, out3 = _both(meta3, slots3, bm3, m, rows.shape[1])
        assert torch.equal(out3, ref3) and torch.equal(out3, src3[:m])
    say("[noalloc] ok")


def test_noalloc_refuses_more_tiles_than_its_scratch():
    raw = _layers(1)
    n, L = raw.shape
    meta, src, slots, bm = _encoded(raw)
    tiles = -(-(L // 4) // 2048)
    too_many = ibp.NOALLOC_MAX_TILES // tiles + 1
    st = ibp.lib().ibp_decompress_noalloc(meta, ctypes.c_void_p(slots.data_ptr()), ctypes.c_void_p(bm.data_ptr()),
                                          too_many, ctypes.c_void_p(src.data_ptr()), None)
    assert st == ibp.IBP_ERR_TOO_LARGE
    assert ibp.status_string(st).startswith("more tiles than")
    assert ibp.ibp_check(meta) == ibp.IBP_OK


def test_noalloc_in_a_graph():
    """Captured once, replayed three times; between the replays an eager
    call on a smaller input reuses the same static scratch."""
    raw = _layers(4)
    n, L = raw.shape
    meta, src, slots, bm = _encoded(raw)
    raw2 = _layers(2, seed=9)
    _, src2, slots2, bm2 = _encoded(raw2, meta)
    dev = device()
    out = torch.empty((n, L), dtype=torch.uint8, device=dev)
    out2 = torch.empty((2, L), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # first call (symbol lookup, launch plans) outside the capture
        ibp.ibp_decompress_noalloc(meta, slots, bm, n, out, stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ibp.ibp_decompress_noalloc(meta, slots, bm, n, out, stream=s)
    for r in range(3):
        out.zero_()
        out2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, src), f"replay {r}"
        ibp.ibp_decompress_noalloc(meta, slots2, bm2, 2, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, src2), f"eager call after replay {r}"
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    say("[noalloc] three replays of a captured call: ok")
