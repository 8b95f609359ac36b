"""Concurrency and capture: one handle used from two streams at once (the
multi-tile look-back and the long-tensor start bits keep their scratch per
stream), and single-tile decode captured in a HIP graph and replayed."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp
from lossless_tensor_compression_ibp_amd import workloads as WL
from tests.gpu_util import as_rows, device, say

pytestmark = pytest.mark.gpu


def test_one_handle_two_streams():
    dev = device()
    # multi-tile tensors: 3 x 64 KiB bf16 rows (look-back per stream)
    layers = [WL.llm_layer(l, rows=32, cols=1024) for l in range(3)]
    raw = np.stack([x.reshape(-1).view(np.uint8) for x in layers])
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    w = WL.LLM_BF16
    meta = ibp.ibp_build_metadata(src, 1, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = torch.empty_like(src)
    bm = torch.zeros(1, dtype=torch.int32, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bm)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs1 = [torch.empty((n, L), dtype=torch.uint8, device=dev) for _ in range(6)]
    outs2 = [torch.empty((n, L), dtype=torch.uint8, device=dev) for _ in range(6)]
    ids = torch.tensor([2, 0, 1], dtype=torch.int64, device=dev)
    for i in range(6):  # interleaved launches on both streams
        with torch.cuda.stream(s1):
            ibp.ibp_decompress(meta, slots, bm, n, outs1[i], stream=s1)
        with torch.cuda.stream(s2):
            ibp.ibp_gather_decompress(meta, slots, n, bm, ids, outs2[i], stream=s2)
    torch.cuda.synchronize()
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    for i in range(6):
        assert torch.equal(outs1[i], src), f"stream 1 launch {i}"
        assert torch.equal(outs2[i], src[ids]), f"stream 2 launch {i}"
    say("[streams] two streams, multi-tile look-back: ok")


def test_multi_tile_encodes_on_two_streams():
    """Long-tensor encodes from HBM (size pass and scan) on one stream and
    from pinned memory (look-back) on another, interleaved through one
    handle: every record equals the one a lone encode writes."""
    dev = device()
    layers = [WL.llm_layer(l, rows=48, cols=1024) for l in range(4)]
    raw = np.stack([x.reshape(-1).view(np.uint8) for x in layers])
    n, L = raw.shape
    src_d = torch.from_numpy(raw).to(dev)
    src_h = torch.from_numpy(raw).pin_memory()
    w = WL.LLM_BF16
    meta = ibp.ibp_build_metadata(src_d, 1, L, w.chunk_bits, w.period_bits, w.threshold)
    ref = torch.empty_like(src_d)
    ref_bm = torch.zeros(1, dtype=torch.int32, device=dev)
    ref_st = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress(meta, src_d, n, ref, ref_bm, ref_st)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {k: [(torch.empty_like(src_d), torch.zeros(1, dtype=torch.int32, device=dev),
                 torch.zeros(n, dtype=torch.int64, device=dev)) for _ in range(5)] for k in ("hbm", "pinned")}
    for i in range(5):
        with torch.cuda.stream(s1):
            sl, bm, st = outs["hbm"][i]
            ibp.ibp_compress(meta, src_d, n, sl, bm, st, stream=s1)
        with torch.cuda.stream(s2):
            sl, bm, st = outs["pinned"][i]
            ibp.ibp_compress(meta, src_h, n, sl, bm, st, stream=s2)
    torch.cuda.synchronize()
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    for k, runs in outs.items():
        for i, (sl, bm, st) in enumerate(runs):
            assert torch.equal(bm, ref_bm) and torch.equal(st, ref_st), f"{k} launch {i}"
            for t in range(n):
                b = int(ref_st[t])
                assert torch.equal(sl[t, :b], ref[t, :b]), f"{k} launch {i}, record {t}"
    say("[streams] two streams, long-tensor encodes from HBM and pinned memory: ok")


def test_single_tile_decode_in_a_graph():
    dev = device()
    w = WL.SPARSE_GNN
    raw = as_rows(WL.sparse_gnn(4096))
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    meta = ibp.ibp_build_metadata(src, 1024, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = torch.empty_like(src)
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bm)
    ids = torch.zeros(1024, dtype=torch.int64, device=dev)
    out = torch.empty((1024, L), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up (launch plans, code objects) outside the capture
        ibp.ibp_gather_decompress(meta, slots, n, bm, ids, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ibp.ibp_gather_decompress(meta, slots, n, bm, ids, out, stream=s)
    rng = np.random.default_rng(4)
    for r in range(5):  # new ids each replay, with eager work and syncs between replays
        new_ids = rng.choice(n, 1024, replace=False)
        ids.copy_(torch.from_numpy(new_ids).to(dev))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, src[torch.from_numpy(new_ids).to(dev)]), f"replay {r}"
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    say("[graph] five replays of a captured gather: ok")


@pytest.mark.parametrize("layout", ["split", "packed"])
def test_layout_gathers_in_a_graph(layout):
    """The gathers of the header-in-GPU-memory layout (pinned slots, as the
    sparse_gnn line) and of the packed HBM cache captured in a HIP graph and
    replayed five times with new ids, eager work and synchronisations between
    the replays; every replay checked against the source rows."""
    dev = device()
    w = WL.SPARSE_GNN
    raw = as_rows(WL.sparse_gnn(4096))
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    meta = ibp.ibp_build_metadata(src, 1024, L, w.chunk_bits, w.period_bits, w.threshold)
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    if layout == "split":
        hw = ibp.header_words(meta)
        slots = torch.empty((n, L), dtype=torch.uint8, pin_memory=True)
        headers = torch.zeros((n, hw), dtype=torch.int32, device=dev)
        ibp.ibp_compress_split(meta, src, n, slots, headers, bm)
    else:
        off = torch.zeros(n + 1, dtype=torch.int64, device=dev)
        ibp.ibp_packed_offsets(meta, src, n, off)
        buf = torch.empty(int(off[-1].item()), dtype=torch.uint8, device=dev)
        ibp.ibp_compress_packed(meta, src, n, off, buf, bm)
    torch.cuda.synchronize()
    ids = torch.zeros(1024, dtype=torch.int64, device=dev)
    out = torch.empty((1024, L), dtype=torch.uint8, device=dev)

    def gather(s):
        if layout == "split":
            ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, ids, out, stream=s)
        else:
            ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, ids, out, stream=s)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up (launch plans, code objects) outside the capture
        gather(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gather(s)
    rng = np.random.default_rng(5)
    for r in range(5):
        new_ids = rng.integers(0, n, 1024)
        ids.copy_(torch.from_numpy(new_ids).to(dev))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, src[torch.from_numpy(new_ids).to(dev)]), f"{layout} replay {r}"
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    say(f"[graph] five replays of a captured {layout} gather: ok")


def test_two_threads_two_handles():
    """Two host threads call the library at the same time, each with its own
    handle and stream: one gathers rows of the header-in-GPU-memory layout,
    the other decodes multi-tile tensors (look-back scratch).  The launch-plan
    cache and the handles' scratch are shared host state; every output is
    checked."""
    import threading

    dev = device()
    w = WL.SPARSE_GNN
    raw_a = as_rows(WL.sparse_gnn(4096))
    na, La = raw_a.shape
    src_a = torch.from_numpy(raw_a).to(dev)
    meta_a = ibp.ibp_build_metadata(src_a, 1024, La, w.chunk_bits, w.period_bits, w.threshold)
    hw = ibp.header_words(meta_a)
    slots_a = torch.empty((na, La), dtype=torch.uint8, pin_memory=True)
    headers = torch.zeros((na, hw), dtype=torch.int32, device=dev)
    bm_a = torch.zeros((na + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress_split(meta_a, src_a, na, slots_a, headers, bm_a)

    wl = WL.LLM_BF16
    raw_b = np.stack([WL.llm_layer(l, rows=48).reshape(-1).view(np.uint8) for l in range(4)])
    nb, Lb = raw_b.shape
    src_b = torch.from_numpy(raw_b).to(dev)
    meta_b = ibp.ibp_build_metadata(src_b, 1, Lb, wl.chunk_bits, wl.period_bits, wl.threshold)
    slots_b = torch.empty_like(src_b)
    bm_b = torch.zeros(1, dtype=torch.int32, device=dev)
    ibp.ibp_compress(meta_b, src_b, nb, slots_b, bm_b)
    torch.cuda.synchronize()

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    rng = np.random.default_rng(6)
    id_sets = [rng.integers(0, na, 2048) for _ in range(20)]
    outs_a = [torch.empty((2048, La), dtype=torch.uint8, device=dev) for _ in range(20)]
    outs_b = [torch.empty((nb, Lb), dtype=torch.uint8, device=dev) for _ in range(20)]
    ids_dev = [torch.from_numpy(x).to(dev) for x in id_sets]
    errors = []
    start = threading.Barrier(2)

    def run_a():
        try:
            start.wait()
            for i in range(20):
                ibp.ibp_gather_decompress_split(meta_a, slots_a, na, headers, bm_a, ids_dev[i], outs_a[i], stream=sa)
            sa.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    def run_b():
        try:
            start.wait()
            for i in range(20):
                ibp.ibp_decompress(meta_b, slots_b, bm_b, nb, outs_b[i], stream=sb)
            sb.synchronize()
        except Exception as e:
            errors.append(e)

    ta, tb = threading.Thread(target=run_a), threading.Thread(target=run_b)
    ta.start()
    tb.start()
    ta.join(timeout=60)
    tb.join(timeout=60)
    assert not ta.is_alive() and not tb.is_alive(), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    assert ibp.ibp_check(meta_a) == ibp.IBP_OK and ibp.ibp_check(meta_b) == ibp.IBP_OK
    for i in range(20):
        assert torch.equal(outs_a[i], src_a[ids_dev[i]]), f"thread A call {i}"
        assert torch.equal(outs_b[i], src_b), f"thread B call {i}"
    say("[threads] two threads, two handles, two streams: ok")


def _three_tile_tensors(n: int = 3):
    """n bf16 tensors of 40 x 256 (20 KiB = 5,120 words): three decode tiles
    of at most 2,048 words and five encode tiles of 1,024, so every call on
    them takes the look-back path."""
    raw = np.stack([WL.llm_layer(l, rows=40, cols=256).reshape(-1).view(np.uint8) for l in range(n)])
    w = WL.LLM_BF16
    return raw, w.chunk_bits, w.period_bits, w.threshold


def test_look_back_calls_refused_under_capture():
    """Multi-tile compress, decompress, gather and the packed offsets scan
    are refused (IBP_ERR_UNSUPPORTED, nothing queued) while the stream
    captures a graph; eager calls on the same stream afterwards are still
    bit-exact against the oracle."""
    from oracle import oracle
    from tests.gpu_util import oracle_metadata

    oracle.build(force=False)
    dev = device()
    raw, W, M, T = _three_tile_tensors()
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    meta = ibp.ibp_build_metadata(src, 1, L, W, M, T)
    om, ob = oracle_metadata(meta, raw[:1], W, M, T)
    o_slots, o_bm, o_st = oracle.compress(raw, L, W, M, om, ob, n)
    assert np.unpackbits(o_bm.view(np.uint8), bitorder="little")[:n].all(), "every tensor compresses"
    slots = torch.empty_like(src)
    bm = torch.zeros(1, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    out = torch.empty_like(src)
    ids = torch.tensor([2, 0, 2], dtype=torch.int64, device=dev)
    gout = torch.empty((3, L), dtype=torch.uint8, device=dev)
    offsets = torch.zeros(n + 1, dtype=torch.int64, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ibp.ibp_compress(meta, src, n, slots, bm, stored, stream=s)  # eager, before the capture
    s.synchronize()
    say("[capture] multi-tile calls under capture")
    refused = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            for name, call in (
                    ("compress", lambda: ibp.ibp_compress(meta, src, n, slots, bm, stored, stream=s)),
                    ("decompress", lambda: ibp.ibp_decompress(meta, slots, bm, n, out, stream=s)),
                    ("gather", lambda: ibp.ibp_gather_decompress(meta, slots, n, bm, ids, gout, stream=s))):
                try:
                    call()
                except ibp.IBPError as e:
                    refused.append((name, e.status))
        finally:
            g.capture_end()
    assert refused == [("compress", ibp.IBP_ERR_UNSUPPORTED), ("decompress", ibp.IBP_ERR_UNSUPPORTED),
                       ("gather", ibp.IBP_ERR_UNSUPPORTED)], refused
    del g
    # packed offsets (look-back scan over item sizes): sparse rows
    ws = WL.SPARSE_GNN
    rows = as_rows(WL.sparse_gnn(600))
    src_s = torch.from_numpy(rows).to(dev)
    meta_s = ibp.ibp_build_metadata(src_s, 600, rows.shape[1], ws.chunk_bits, ws.period_bits, ws.threshold)
    off_s = torch.zeros(601, dtype=torch.int64, device=dev)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g2.capture_begin()
        try:
            with pytest.raises(ibp.IBPError) as e:
                ibp.ibp_packed_offsets(meta_s, src_s, 600, off_s, stream=s)
        finally:
            g2.capture_end()
    assert e.value.status == ibp.IBP_ERR_UNSUPPORTED
    del g2
    # eager calls on the same stream: bit-exact against the oracle
    with torch.cuda.stream(s):
        slots.fill_(0xEE)
        ibp.ibp_compress(meta, src, n, slots, bm, stored, stream=s)
        ibp.ibp_decompress(meta, torch.from_numpy(o_slots).to(dev), torch.from_numpy(o_bm.view(np.int32).copy()).to(dev),
                           n, out, stream=s)
        ibp.ibp_gather_decompress(meta, slots, n, bm, ids, gout, stream=s)
        ibp.ibp_packed_offsets(meta_s, src_s, 600, off_s, stream=s)
    s.synchronize()
    assert ibp.ibp_check(meta, stream=s) == ibp.IBP_OK and ibp.ibp_check(meta_s, stream=s) == ibp.IBP_OK
    st = stored.cpu().numpy().astype(np.uint64)
    np.testing.assert_array_equal(st, o_st)
    sl = slots.cpu().numpy()
    for t in range(n):
        k = int(o_st[t])
        assert np.array_equal(sl[t, :k], o_slots[t, :k]), f"record {t} differs from the oracle's"
    np.testing.assert_array_equal(out.cpu().numpy(), raw)
    np.testing.assert_array_equal(gout.cpu().numpy(), raw[[2, 0, 2]])
    om_s, ob_s = oracle_metadata(meta_s, rows, ws.chunk_bits, ws.period_bits, ws.threshold)
    o_off = oracle.packed_offsets(rows, rows.shape[1], ws.chunk_bits, ws.period_bits, om_s, ob_s, 600)
    np.testing.assert_array_equal(off_s.cpu().numpy().astype(np.uint64), o_off)
    say("[capture] refused under capture, eager calls afterwards bit-exact: ok")


def test_one_stream_two_threads_look_back():
    """Two host threads queue multi-tile calls on ONE stream through one
    handle (so they share its look-back scratch): thread A decodes and
    gathers, thread B compresses into its own slots.  Every output is checked
    against the source and the first compress."""
    import threading

    dev = device()
    raw, W, M, T = _three_tile_tensors(4)
    n, L = raw.shape
    src = torch.from_numpy(raw).to(dev)
    meta = ibp.ibp_build_metadata(src, 1, L, W, M, T)
    slots = torch.empty_like(src)
    bm = torch.zeros(1, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bm, stored)
    torch.cuda.synchronize()
    st_ref = stored.cpu().numpy()
    s = torch.cuda.Stream()
    k = 20
    rng = np.random.default_rng(11)
    id_sets = [torch.from_numpy(rng.integers(0, n, 5)).to(dev) for _ in range(k)]
    outs_a = [torch.empty((n, L), dtype=torch.uint8, device=dev) for _ in range(k)]
    gouts_a = [torch.empty((5, L), dtype=torch.uint8, device=dev) for _ in range(k)]
    slots_b = [torch.empty_like(src) for _ in range(k)]
    bms_b = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(k)]
    sts_b = [torch.zeros(n, dtype=torch.int64, device=dev) for _ in range(k)]
    errors = []
    start = threading.Barrier(2)

    def run_a():
        try:
            start.wait()
            for i in range(k):
                ibp.ibp_decompress(meta, slots, bm, n, outs_a[i], stream=s)
                ibp.ibp_gather_decompress(meta, slots, n, bm, id_sets[i], gouts_a[i], stream=s)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    def run_b():
        try:
            start.wait()
            for i in range(k):
                ibp.ibp_compress(meta, src, n, slots_b[i], bms_b[i], sts_b[i], stream=s)
        except Exception as e:
            errors.append(e)

    say("[threads] two threads, one stream, multi-tile look-back")
    ta, tb = threading.Thread(target=run_a), threading.Thread(target=run_b)
    ta.start()
    tb.start()
    ta.join(timeout=60)
    tb.join(timeout=60)
    assert not ta.is_alive() and not tb.is_alive(), "a thread did not finish"
    assert not errors, errors
    s.synchronize()
    assert ibp.ibp_check(meta, stream=s) == ibp.IBP_OK
    ref = slots.cpu().numpy()
    for i in range(k):
        assert torch.equal(outs_a[i], src), f"decode {i}"
        assert torch.equal(gouts_a[i], src[id_sets[i]]), f"gather {i}"
        assert torch.equal(bms_b[i], bm), f"bitmask of compress {i}"
        np.testing.assert_array_equal(sts_b[i].cpu().numpy(), st_ref)
        sb = slots_b[i].cpu().numpy()
        for t in range(n):
            assert np.array_equal(sb[t, :st_ref[t]], ref[t, :st_ref[t]]), f"compress {i}, record {t}"
    say("[threads] two threads, one stream: ok")
