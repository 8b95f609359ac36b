"""GPU parity of the packed cache layout (items back to back on 16-byte
boundaries; FR/KO summary, "Intégration au système", software cache): the
HIP path through the C ABI against the oracle, bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp
from lossless_tensor_compression_ibp_amd import workloads as WL
from oracle import oracle
from tests.gpu_util import as_rows, device, oracle_metadata, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def _rows(wl: str, n: int) -> np.ndarray:
    if wl == "sparse_gnn":
        return as_rows(WL.sparse_gnn(n))
    if wl == "dense_gnn":
        return as_rows(WL.dense_gnn(n))
    if wl == "dlrm":
        return as_rows(WL.dlrm(n))
    kv = WL.kv_cache(n_layers=1, n_heads=1, n_tokens=16 * n)
    return kv.reshape(-1, 2048).view(np.uint8).reshape(-1, 4096)


def packed_case(raw: np.ndarray, W: int, M: int, T: float, n_sample: int, *, src_pinned=False, buf_pinned=False,
                label=""):
    n, L = raw.shape
    dev = device()
    say(f"[packed] {label} n={n} L={L} W={W} M={M} src_pinned={src_pinned} buf_pinned={buf_pinned}")
    src = to_gpu(raw, pinned=src_pinned)
    meta = ibp.ibp_build_metadata(src, n_sample, L, W, M, T)
    om, ob = oracle_metadata(meta, raw[:n_sample], W, M, T)
    # offsets
    off = torch.full((n + 1,), -1, dtype=torch.int64, device=dev)
    ibp.ibp_packed_offsets(meta, src, n, off)
    o_buf, o_off, o_bm = oracle.compress_packed(raw, L, W, M, om, ob, n)
    np.testing.assert_array_equal(off.cpu().numpy().astype(np.uint64), o_off, err_msg="offsets differ")
    total = int(o_off[-1])
    # items
    cap = total + 64
    if buf_pinned:
        buf = torch.full((cap,), 0xEE, dtype=torch.uint8, pin_memory=True)
    else:
        buf = torch.full((cap,), 0xEE, dtype=torch.uint8, device=dev)
    bm = torch.zeros(max(1, (n + 31) // 32), dtype=torch.int32, device=dev)
    ibp.ibp_compress_packed(meta, src, n, off, buf, bm, capacity=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(buf.cpu().numpy()[:total], o_buf[:total], err_msg="packed bytes differ")
    assert (buf.cpu().numpy()[total:] == 0xEE).all(), "wrote past the last item"
    np.testing.assert_array_equal(bm.cpu().numpy().view(np.uint32)[: o_bm.size], o_bm, err_msg="bitmask differs")
    # decode: GPU buffer, and the oracle's buffer decoded by the GPU
    out = torch.empty((n, L), dtype=torch.uint8, device=dev)
    ibp.ibp_decompress_packed(meta, buf, off, bm, n, out, buf_bytes=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out.cpu().numpy(), raw)
    obuf_t = torch.from_numpy(np.ascontiguousarray(o_buf[:total])).to(dev)
    obm_t = torch.from_numpy(o_bm.view(np.int32).copy()).to(dev) if o_bm.size else bm
    out2 = torch.empty_like(out)
    ibp.ibp_decompress_packed(meta, obuf_t, off, obm_t, n, out2)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out2.cpu().numpy(), raw)
    ids = np.random.default_rng(n).integers(0, n, size=2 * n + 5)
    g = torch.empty((ids.size, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.from_numpy(ids).to(dev), g, buf_bytes=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(g.cpu().numpy(), raw[ids])
    say(f"[packed] {label} ok: {total} bytes for {n * L} ({n * L / max(total, 1):.3f}x)")
    return meta, src, off, buf, bm, cap


@pytest.mark.parametrize("wl,n", [("sparse_gnn", 2500), ("dense_gnn", 1500), ("dlrm", 3000), ("kv_bf16", 600)])
def test_packed_workload_shapes(wl, n):
    w = WL.ALL[wl]
    raw = _rows(wl, n)
    packed_case(raw, w.chunk_bits, w.period_bits, w.threshold, min(n, w.n_sample), label=wl)


def test_packed_pinned_buffer_and_source():
    w = WL.SPARSE_GNN
    raw = _rows("sparse_gnn", 1200)
    packed_case(raw, w.chunk_bits, w.period_bits, w.threshold, 1024, src_pinned=True, buf_pinned=True,
                label="sparse pinned")


@pytest.mark.parametrize("W,M,L,n", [(32, 32, 64, 70), (64, 512, 256, 129), (1024, 1024, 128, 33),
                                     (32, 32, 8192, 20), (256, 2048, 1024, 65)])
def test_packed_shapes_and_edges(W, M, L, n):
    rng = np.random.default_rng(W * 7 + L)
    base = rng.integers(0, 2**32, size=L // 4, dtype=np.uint64).astype(np.uint32)
    rows = np.tile(base, (n, 1)) ^ rng.integers(0, 2**12, size=(n, L // 4), dtype=np.uint64).astype(np.uint32)
    rows[::5] = rng.integers(0, 2**32, size=rows[::5].shape, dtype=np.uint64).astype(np.uint32)  # raw items
    packed_case(rows.view(np.uint8).reshape(n, L), W, M, 0.9, n, label=f"W={W} M={M} L={L}")


@pytest.mark.parametrize("W,M,L", [(32, 32, 64), (64, 512, 256)], ids=["uniform", "per_position"])
def test_packed_past_the_row_kernel_bound(W, M, L):
    """More items than 128 per CU: the decode of all items and the gather of
    2n + 5 ids take the persistent kernel, smaller launches one wave per row."""
    rng = np.random.default_rng(L)
    n = 128 * torch.cuda.get_device_properties(0).multi_processor_count + 37
    base = rng.integers(0, 2**32, size=L // 4, dtype=np.uint64).astype(np.uint32)
    rows = np.tile(base, (n, 1)) ^ rng.integers(0, 2**12, size=(n, L // 4), dtype=np.uint64).astype(np.uint32)
    rows[::5] = rng.integers(0, 2**32, size=rows[::5].shape, dtype=np.uint64).astype(np.uint32)
    meta, src, off, buf, bm, cap = packed_case(rows.view(np.uint8).reshape(n, L), W, M, 0.9, 1024,
                                               label=f"past the row bound W={W} M={M} L={L}")
    ids = rng.integers(0, n, 3000)
    g = torch.empty((ids.size, L), dtype=torch.uint8, device=device())
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.from_numpy(ids).to(device()), g, buf_bytes=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(g.cpu().numpy(), rows.view(np.uint8).reshape(n, L)[ids])


@pytest.mark.parametrize("wl", ["dense_gnn", "sparse_gnn"])
def test_packed_errors(wl):
    """dense_gnn has per-position metadata (the persistent kernel), sparse_gnn
    the same word at every position (one wave per gathered row)."""
    w = WL.ALL[wl]
    raw = _rows(wl, 300)
    n, L = raw.shape
    dev = device()
    meta, src, off, buf, bm, cap = packed_case(raw, w.chunk_bits, w.period_bits, w.threshold, 300,
                                               label=f"errors {wl}")
    total = int(off[-1].item())
    # capacity one item short: the last item is not written, range error
    small = torch.full((total,), 0xEE, dtype=torch.uint8, device=dev)
    ibp.ibp_compress_packed(meta, src, n, off, small, bm, capacity=total - 16)
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_RANGE
    last = int(off[-2].item())
    assert (small.cpu().numpy()[last:] == 0xEE).all()
    # offsets that do not match the data: corrupt, nothing written there
    bad = off.clone()
    bad[1] += 16
    ibp.ibp_compress_packed(meta, src, n, bad, small, bm, capacity=total)
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    # decode: an id out of range, an item cut short, a misaligned offset
    out = torch.empty((4, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.tensor([0, n, 1, 2], device=dev), out)
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_RANGE
    comp = np.unpackbits(bm.cpu().numpy().view(np.uint8), bitorder="little")[:n].astype(bool)
    sizes = np.diff(off.cpu().numpy())
    t = int(np.nonzero(comp & (sizes > 16))[0][0])
    bad = off.clone()
    bad[t + 1] = bad[t] + 16  # 16 bytes cannot hold this record
    ibp.ibp_gather_decompress_packed(meta, buf, bad, n, bm, torch.tensor([t], device=dev), out[:1])
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    bad = off.clone()
    bad[t] += 4
    ibp.ibp_gather_decompress_packed(meta, buf, bad, n, bm, torch.tensor([t], device=dev), out[:1])
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    # a raw item cut shorter than the tensor
    raw_ids = np.nonzero(~comp)[0]
    if raw_ids.size:
        r = int(raw_ids[0])
        bad = off.clone()
        bad[r + 1] = bad[r] + L - 16
        ibp.ibp_gather_decompress_packed(meta, buf, bad, n, bm, torch.tensor([r], device=dev), out[:1])
        assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    # offsets past the buffer
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.tensor([n - 1], device=dev), out[:1],
                                     buf_bytes=int(off[-2].item()))
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    # the handle still works afterwards
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.tensor([n - 1, 0], device=dev), out[:2])
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out[:2].cpu().numpy(), raw[[n - 1, 0]])


def test_packed_empty_and_unsupported():
    dev = device()
    w = WL.DENSE_GNN
    raw = _rows("dense_gnn", 64)
    src = to_gpu(raw)
    meta = ibp.ibp_build_metadata(src, 64, raw.shape[1], w.chunk_bits, w.period_bits, w.threshold)
    off = torch.full((1,), -1, dtype=torch.int64, device=dev)
    ibp.ibp_packed_offsets(meta, src, 0, off)
    torch.cuda.synchronize()
    assert int(off[0].item()) == 0
    # a multi-tile tensor (more than 8 KiB) has no packed path
    big = torch.zeros((2, 8192 + 16), dtype=torch.uint8, device=dev)
    m2 = ibp.ibp_build_metadata(big, 2, 8192 + 16, 32, 32, 0.95)
    off2 = torch.zeros(3, dtype=torch.int64, device=dev)
    with pytest.raises(ibp.IBPError) as e:
        ibp.ibp_packed_offsets(m2, big, 2, off2)
    assert e.value.status == ibp.IBP_ERR_UNSUPPORTED


@pytest.mark.timeout(600)
def test_packed_sparse_gnn_full_size():
    """All 1,048,576 rows packed into HBM; sampled items against the oracle,
    gathers of 8,192 distinct ids against the source."""
    w = WL.SPARSE_GNN
    n, L = w.n_tensors, w.tensor_bytes
    dev = device()
    say(f"[packed] sparse_gnn full n={n}")
    host = torch.empty((n, L), dtype=torch.uint8, pin_memory=True)
    WL.sparse_gnn(n, out=host.numpy().view(np.float32).reshape(n, 256))
    raw = host.numpy()
    meta = ibp.ibp_build_metadata(host, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    off = torch.empty(n + 1, dtype=torch.int64, device=dev)
    ibp.ibp_packed_offsets(meta, host, n, off)
    off_np = off.cpu().numpy().astype(np.uint64)
    total = int(off_np[-1])
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress_packed(meta, host, n, off, buf, bm)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    om, ob = oracle_metadata(meta, raw[: w.n_sample], w.chunk_bits, w.period_bits, w.threshold)
    rows = np.unique(np.concatenate([np.arange(300), np.random.default_rng(9).integers(0, n, 1500), [n - 1]]))
    sizes = np.diff(off_np.astype(np.int64))
    bnp = buf.cpu().numpy()
    for r in rows:
        o_buf, o_off, _ = oracle.compress_packed(raw[r:r + 1], L, w.chunk_bits, w.period_bits, om, ob, 1)
        assert sizes[r] == int(o_off[1]), f"item size of row {r}"
        a = int(off_np[r])
        assert np.array_equal(bnp[a:a + sizes[r]], o_buf[: sizes[r]]), f"item of row {r}"
    ids_all = WL.batch_ids(n, 8192, 3, replace=False)
    out = torch.empty((8192, L), dtype=torch.uint8, device=dev)
    for i in range(ids_all.shape[0]):
        ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.from_numpy(ids_all[i]).to(dev), out)
        assert ibp.ibp_check(meta) == ibp.IBP_OK
        np.testing.assert_array_equal(out.cpu().numpy(), raw[ids_all[i]])
    say(f"[packed] sparse_gnn full ok: {total} bytes for {n * L} ({n * L / total:.3f}x capacity)")
