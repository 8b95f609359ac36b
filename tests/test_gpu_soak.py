"""Soak of every decode and encode path (opt-in: set IBP_SOAK_SECONDS).

Repeats, until the time is spent: the decode of KV pages in HBM, gathers of
header-in-GPU-memory rows from pinned slots, of the packed HBM cache and of
512-byte rows in HBM, the multi-tile (look-back) decode of layers from pinned
slots; and the encodes of KV pages, dense rows, multi-tile layers (from HBM
and from pinned memory), headers in GPU memory and the packed cache.  Every
decoded output must equal its source, and every repetition of an encode must
give the first run's bitmask and stored bytes (or offsets) and decode
exactly.  Races between waves (look-back, bitmask words, persistent
pipelines) that a single pass could miss would show up as a mismatch."""
from __future__ import annotations

import os
import time

import numpy as np
import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp
from lossless_tensor_compression_ibp_amd import workloads as WL
from tests.gpu_util import device, say

SOAK_S = float(os.environ.get("IBP_SOAK_SECONDS", "0"))
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(int(SOAK_S * 2) + 300),
              pytest.mark.skipif(SOAK_S <= 0, reason="opt-in soak: set IBP_SOAK_SECONDS")]


def _rows(x: np.ndarray, dev) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x.view(np.uint8).reshape(x.shape[0], -1)).to(dev)


def test_soak_decode_paths():
    dev = device()
    w = WL.KV_BF16
    kv = WL.kv_cache(n_layers=8)
    src_kv = torch.from_numpy(kv.reshape(-1, 2048).view(np.uint8).reshape(-1, 4096)).to(dev)
    n_kv = src_kv.shape[0]
    m_kv = ibp.ibp_build_metadata(src_kv, w.n_sample, 4096, w.chunk_bits, w.period_bits, w.threshold)
    sl_kv = torch.empty_like(src_kv)
    bm_kv = torch.zeros((n_kv + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress(m_kv, src_kv, n_kv, sl_kv, bm_kv)
    out_kv = torch.empty_like(src_kv)
    w = WL.SPARSE_GNN
    n_sp = 262144
    src_sp = _rows(WL.sparse_gnn(n_sp), dev)
    m_sp = ibp.ibp_build_metadata(src_sp, 1024, 1024, w.chunk_bits, w.period_bits, w.threshold)
    hw = ibp.header_words(m_sp)
    sl_sp = torch.empty((n_sp, 1024), dtype=torch.uint8, pin_memory=True)
    hd_sp = torch.zeros((n_sp, hw), dtype=torch.int32, device=dev)
    bm_sp = torch.zeros((n_sp + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress_split(m_sp, src_sp, n_sp, sl_sp, hd_sp, bm_sp)
    off = torch.zeros(n_sp + 1, dtype=torch.int64, device=dev)
    ibp.ibp_packed_offsets(m_sp, src_sp, n_sp, off)
    buf = torch.empty(int(off[-1].item()), dtype=torch.uint8, device=dev)
    bm_pk = torch.zeros_like(bm_sp)
    ibp.ibp_compress_packed(m_sp, src_sp, n_sp, off, buf, bm_pk)
    w = WL.LLM_BF16
    src_ll = torch.from_numpy(np.stack([WL.llm_layer(l, rows=512).reshape(-1).view(np.uint8)
                                        for l in range(4)])).to(dev)
    n_ll, L_ll = src_ll.shape
    m_ll = ibp.ibp_build_metadata(src_ll, 1, L_ll, w.chunk_bits, w.period_bits, w.threshold)
    sl_ll = torch.empty((n_ll, L_ll), dtype=torch.uint8, pin_memory=True)
    bm_ll = torch.zeros(1, dtype=torch.int32, device=dev)
    ibp.ibp_compress(m_ll, src_ll, n_ll, sl_ll, bm_ll)
    out_ll = torch.empty_like(src_ll)
    # 512-byte rows (the two-words-per-lane stage) in HBM, gathered with repeats
    w = WL.DENSE_GNN
    src_dg = _rows(WL.dense_gnn(16384), dev)
    n_dg = src_dg.shape[0]
    m_dg = ibp.ibp_build_metadata(src_dg, 1024, 512, w.chunk_bits, w.period_bits, w.threshold)
    sl_dg = torch.empty_like(src_dg)
    bm_dg = torch.zeros((n_dg + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_compress(m_dg, src_dg, n_dg, sl_dg, bm_dg)
    out_dg = torch.empty((8192, 512), dtype=torch.uint8, device=dev)
    out_sp = torch.empty((8192, 1024), dtype=torch.uint8, device=dev)
    out_pk = torch.empty_like(out_sp)
    g = torch.Generator(device=dev).manual_seed(9)
    it, t0, last = 0, time.time(), time.time()
    while time.time() - t0 < SOAK_S:
        ids = torch.randint(0, n_sp, (8192,), device=dev, generator=g)
        ibp.ibp_decompress(m_kv, sl_kv, bm_kv, n_kv, out_kv)
        ibp.ibp_gather_decompress_split(m_sp, sl_sp, n_sp, hd_sp, bm_sp, ids, out_sp)
        ibp.ibp_gather_decompress_packed(m_sp, buf, off, n_sp, bm_pk, ids, out_pk)
        ibp.ibp_decompress(m_ll, sl_ll, bm_ll, n_ll, out_ll)
        ids_dg = ids % n_dg
        ibp.ibp_gather_decompress(m_dg, sl_dg, n_dg, bm_dg, ids_dg, out_dg)
        assert torch.equal(out_kv, src_kv), f"KV pages, iteration {it}"
        assert torch.equal(out_dg, src_dg[ids_dg]), f"512-byte rows, iteration {it}"
        assert torch.equal(out_sp, src_sp[ids]), f"split gather, iteration {it}"
        assert torch.equal(out_pk, src_sp[ids]), f"packed gather, iteration {it}"
        assert torch.equal(out_ll, src_ll), f"multi-tile layers, iteration {it}"
        it += 1
        if time.time() - last > 20:
            last = time.time()
            say(f"[soak decode] {it} iterations exact after {last - t0:.0f} s")
    for m in (m_kv, m_sp, m_ll, m_dg):
        assert ibp.ibp_check(m) == ibp.IBP_OK
    say(f"[soak decode] {it} iterations of 5 decodes, all exact")


def test_soak_encode_paths():
    dev = device()
    w = WL.KV_BF16
    kv = WL.kv_cache(n_layers=4)
    src_kv = torch.from_numpy(kv.reshape(-1, 2048).view(np.uint8).reshape(-1, 4096)).to(dev)
    m_kv = ibp.ibp_build_metadata(src_kv, w.n_sample, 4096, w.chunk_bits, w.period_bits, w.threshold)
    w = WL.DENSE_GNN
    src_dg = _rows(WL.dense_gnn(16384), dev)
    m_dg = ibp.ibp_build_metadata(src_dg, 1024, 512, w.chunk_bits, w.period_bits, w.threshold)
    w = WL.LLM_BF16
    src_ll = torch.from_numpy(np.stack([WL.llm_layer(l, rows=256).reshape(-1).view(np.uint8)
                                        for l in range(3)])).to(dev)
    m_ll = ibp.ibp_build_metadata(src_ll, 1, src_ll.shape[1], w.chunk_bits, w.period_bits, w.threshold)
    w = WL.SPARSE_GNN
    src_sp = _rows(WL.sparse_gnn(65536), dev)
    m_sp = ibp.ibp_build_metadata(src_sp, 1024, 1024, w.chunk_bits, w.period_bits, w.threshold)
    hw = ibp.header_words(m_sp)

    def bitmask(n):
        return torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)

    def enc_plain(m, src):
        # slots and output in HBM whether the source is in HBM or pinned
        n = src.shape[0]
        sl = torch.empty(src.shape, dtype=src.dtype, device=dev)
        bm, st = bitmask(n), torch.zeros(n, dtype=torch.int64, device=dev)
        ibp.ibp_compress(m, src, n, sl, bm, st)
        out = torch.empty(src.shape, dtype=src.dtype, device=dev)
        ibp.ibp_decompress(m, sl, bm, n, out)
        return bm, st, torch.equal(out.cpu(), src.cpu()) if src.device.type == "cpu" else torch.equal(out, src)

    def enc_split(m, src):
        n = src.shape[0]
        sl, bm, st = torch.empty_like(src), bitmask(n), torch.zeros(n, dtype=torch.int64, device=dev)
        hd = torch.zeros((n, hw), dtype=torch.int32, device=dev)
        ibp.ibp_compress_split(m, src, n, sl, hd, bm, st)
        out = torch.empty_like(src)
        ibp.ibp_decompress_split(m, sl, hd, bm, n, out)
        return bm, st, torch.equal(out, src)

    def enc_packed(m, src):
        n = src.shape[0]
        off = torch.zeros(n + 1, dtype=torch.int64, device=dev)
        ibp.ibp_packed_offsets(m, src, n, off)
        buf, bm = torch.empty(int(off[-1].item()), dtype=torch.uint8, device=dev), bitmask(n)
        ibp.ibp_compress_packed(m, src, n, off, buf, bm)
        out = torch.empty_like(src)
        ibp.ibp_decompress_packed(m, buf, off, bm, n, out)
        return bm, off, torch.equal(out, src)

    src_ll_pinned = src_ll.cpu().pin_memory()  # long tensors: look-back from pinned memory, two passes from HBM
    cases = [("kv", enc_plain, m_kv, src_kv), ("dense", enc_plain, m_dg, src_dg), ("llm", enc_plain, m_ll, src_ll),
             ("llm_pinned_source", enc_plain, m_ll, src_ll_pinned),
             ("split", enc_split, m_sp, src_sp), ("packed", enc_packed, m_sp, src_sp)]
    first = {name: f(m, s) for name, f, m, s in cases}
    assert all(v[2] for v in first.values()), "a first encode does not round-trip"
    it, t0, last = 0, time.time(), time.time()
    while time.time() - t0 < SOAK_S:
        for name, f, m, s in cases:
            bm, st, ok = f(m, s)
            assert ok, f"{name}: decode differs, iteration {it}"
            assert torch.equal(bm, first[name][0]) and torch.equal(st, first[name][1]), f"{name}, iteration {it}"
        it += 1
        if time.time() - last > 20:
            last = time.time()
            say(f"[soak encode] {it} iterations exact after {last - t0:.0f} s")
    for m in (m_kv, m_dg, m_ll, m_sp):
        assert ibp.ibp_check(m) == ibp.IBP_OK
    say(f"[soak encode] {it} iterations of {len(cases)} encodes, all exact")
