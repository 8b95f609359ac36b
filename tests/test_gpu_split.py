"""GPU parity of the header-in-GPU-memory slot layout (FR/KO summary,
"Intégration au système": GPU-resident bitmask, here with the header words
beside it): the HIP path through the C ABI against the oracle, bit for bit."""
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


def split_case(raw: np.ndarray, W: int, M: int, T: float, n_sample: int, *, pinned=False, label=""):
    n, L = raw.shape
    dev = device()
    hw = oracle.header_words(L, W)
    say(f"[split] {label} n={n} L={L} W={W} M={M} hw={hw} pinned={pinned}")
    src = to_gpu(raw, pinned=pinned)
    meta = ibp.ibp_build_metadata(src, n_sample, L, W, M, T)
    om, ob = oracle_metadata(meta, raw[:n_sample], W, M, T)
    if pinned:
        slots = torch.full((n, L), 0xEE, dtype=torch.uint8, pin_memory=True)
    else:
        slots = torch.full((n, L), 0xEE, dtype=torch.uint8, device=dev)
    headers = torch.full((n, hw), -1, dtype=torch.int32, device=dev)
    bm = torch.zeros(max(1, (n + 31) // 32), dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress_split(meta, src, n, slots, headers, bm, stored)
    torch.cuda.synchronize()
    o_slots, o_hdr, o_bm, o_st = oracle.compress_split(raw, L, W, M, om, ob, n)
    np.testing.assert_array_equal(bm.cpu().numpy().view(np.uint32)[: o_bm.size], o_bm, err_msg="bitmask")
    np.testing.assert_array_equal(headers.cpu().numpy().view(np.uint32), o_hdr, err_msg="headers")
    st = stored.cpu().numpy().astype(np.uint64)
    np.testing.assert_array_equal(st, o_st, err_msg="stored bytes")
    sl = slots.cpu().numpy()
    for t in range(n):
        k = int(st[t])
        if not np.array_equal(sl[t, :k], o_slots[t, :k]):
            raise AssertionError(f"slot {t} differs from the oracle's")
    # decode the GPU's and the oracle's slots
    out = torch.empty((n, L), dtype=torch.uint8, device=dev)
    ibp.ibp_decompress_split(meta, slots, headers, bm, n, out)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out.cpu().numpy(), raw)
    oslots_t = to_gpu(o_slots, pinned=pinned)
    ohdr_t = torch.from_numpy(o_hdr.view(np.int32).copy()).to(dev)
    obm_t = torch.from_numpy(o_bm.view(np.int32).copy()).to(dev)
    out2 = torch.empty_like(out)
    ibp.ibp_decompress_split(meta, oslots_t, ohdr_t, obm_t, n, out2)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out2.cpu().numpy(), raw)
    ids = np.random.default_rng(n + L).integers(0, n, size=2 * n + 3)
    g = torch.empty((ids.size, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, torch.from_numpy(ids).to(dev), g)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(g.cpu().numpy(), raw[ids])
    ncomp = int(np.unpackbits(o_bm.view(np.uint8), bitorder="little")[:n].sum())
    say(f"[split] {label} ok ({ncomp} of {n} compressed)")
    return meta, slots, headers, bm


@pytest.mark.parametrize("wl,n,pinned", [("sparse_gnn", 2500, True), ("dense_gnn", 1500, False),
                                         ("dlrm", 3000, True)])
def test_split_workload_shapes(wl, n, pinned):
    w = WL.ALL[wl]
    gen = {"sparse_gnn": WL.sparse_gnn, "dense_gnn": WL.dense_gnn, "dlrm": WL.dlrm}[wl]
    raw = as_rows(gen(n))
    split_case(raw, w.chunk_bits, w.period_bits, w.threshold, min(n, 1024), pinned=pinned, label=wl)


@pytest.mark.parametrize("W,M,L,n", [(32, 32, 64, 70), (64, 512, 256, 129), (1024, 1024, 128, 33),
                                     (256, 2048, 1024, 65), (32, 4096, 512, 90), (128, 128, 2048, 40)])
def test_split_shapes(W, M, L, n):
    rng = np.random.default_rng(W * 3 + L)
    base = rng.integers(0, 2**32, size=L // 4, dtype=np.uint64).astype(np.uint32)
    rows = np.tile(base, (n, 1)) ^ rng.integers(0, 2**12, size=(n, L // 4), dtype=np.uint64).astype(np.uint32)
    rows[::7] = rng.integers(0, 2**32, size=rows[::7].shape, dtype=np.uint64).astype(np.uint32)
    split_case(rows.view(np.uint8).reshape(n, L), W, M, 0.9, n, label=f"W={W} M={M} L={L}")


def test_split_errors_and_unsupported():
    w = WL.DENSE_GNN
    raw = as_rows(WL.dense_gnn(200))
    n, L = raw.shape
    dev = device()
    meta, slots, headers, bm = split_case(raw, w.chunk_bits, w.period_bits, w.threshold, 200, label="errors")
    out = torch.empty((3, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, torch.tensor([0, n, 1], device=dev), out)
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_RANGE
    comp = np.nonzero(np.unpackbits(bm.cpu().numpy().view(np.uint8), bitorder="little")[:n])[0]
    t = int(comp[0])
    bad = headers.clone()
    bad[t] = 0  # every chunk verbatim: the record would not be shorter than the slot
    ibp.ibp_gather_decompress_split(meta, slots, n, bad, bm, torch.tensor([t], device=dev), out[:1])
    assert ibp.ibp_check(meta) == ibp.IBP_ERR_CORRUPT
    ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, torch.tensor([t, 0], device=dev), out[:2])
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out[:2].cpu().numpy(), raw[[t, 0]])
    # header padding bits set (sparse_gnn: 8 chunks in one header word)
    ws = WL.SPARSE_GNN
    raw2 = as_rows(WL.sparse_gnn(300))
    meta2, slots2, hdr2, bm2 = split_case(raw2, ws.chunk_bits, ws.period_bits, ws.threshold, 300, label="pad")
    comp2 = np.nonzero(np.unpackbits(bm2.cpu().numpy().view(np.uint8), bitorder="little")[:300])[0]
    t2 = int(comp2[0])
    bad2 = hdr2.clone()
    bad2[t2, 0] |= 1 << 20
    out2 = torch.empty((1, 1024), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_split(meta2, slots2, 300, bad2, bm2, torch.tensor([t2], device=dev), out2)
    assert ibp.ibp_check(meta2) == ibp.IBP_ERR_CORRUPT
    # 1,024 chunks per page: 32 header words, beyond this layout
    kv = WL.kv_cache(n_layers=1, n_heads=1, n_tokens=16 * 8).reshape(-1, 2048).view(np.uint8).reshape(-1, 4096)
    src = to_gpu(kv)
    m3 = ibp.ibp_build_metadata(src, 8, 4096, 32, 32768, 0.95)
    with pytest.raises(ibp.IBPError) as e:
        ibp.ibp_compress_split(m3, src, 8, torch.empty_like(src), torch.zeros((8, 32), dtype=torch.int32, device=dev),
                               torch.zeros(1, dtype=torch.int32, device=dev))
    assert e.value.status == ibp.IBP_ERR_UNSUPPORTED


@pytest.mark.timeout(600)
def test_split_sparse_gnn_full_size():
    """All 1,048,576 rows in pinned slots with headers in HBM; sampled slots
    against the oracle, gathers of 8,192 distinct ids against the source."""
    w = WL.SPARSE_GNN
    n, L = w.n_tensors, w.tensor_bytes
    dev = device()
    say(f"[split] sparse_gnn full n={n}")
    host = torch.empty((n, L), dtype=torch.uint8, pin_memory=True)
    WL.sparse_gnn(n, out=host.numpy().view(np.float32).reshape(n, 256))
    raw = host.numpy()
    meta = ibp.ibp_build_metadata(host, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = torch.empty((n, L), dtype=torch.uint8, pin_memory=True)
    headers = torch.empty((n, 1), dtype=torch.int32, device=dev)
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress_split(meta, host, n, slots, headers, bm, stored)
    torch.cuda.synchronize()
    om, ob = oracle_metadata(meta, raw[: w.n_sample], w.chunk_bits, w.period_bits, w.threshold)
    rows = np.unique(np.concatenate([np.arange(256), np.random.default_rng(8).integers(0, n, 2048), [n - 1]]))
    o_slots, o_hdr, o_bm, o_st = oracle.compress_split(raw[rows], L, w.chunk_bits, w.period_bits, om, ob, len(rows))
    st = stored.cpu().numpy().astype(np.uint64)
    hd = headers.cpu().numpy().view(np.uint32)
    bits = (bm.cpu().numpy().view(np.uint32)[rows >> 5] >> (rows & 31)) & 1
    np.testing.assert_array_equal(bits, np.unpackbits(o_bm.view(np.uint8), bitorder="little")[: len(rows)])
    np.testing.assert_array_equal(st[rows], o_st)
    np.testing.assert_array_equal(hd[rows], o_hdr)
    sv = slots.numpy()
    for i, r in enumerate(rows):
        k = int(o_st[i])
        assert np.array_equal(sv[r, :k], o_slots[i, :k]), f"slot {r}"
    ids_all = WL.batch_ids(n, 8192, 3, replace=False)
    out = torch.empty((8192, L), dtype=torch.uint8, device=dev)
    for i in range(ids_all.shape[0]):
        ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, torch.from_numpy(ids_all[i]).to(dev), out)
        assert ibp.ibp_check(meta) == ibp.IBP_OK
        np.testing.assert_array_equal(out.cpu().numpy(), raw[ids_all[i]])
    say("[split] sparse_gnn full ok")
