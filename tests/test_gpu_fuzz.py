"""Seeded random formats against the oracle, bit for bit: chunk widths 32 to
1024, periods, tensor lengths (one tile, several, and several groups of eight
tiles; 16-byte multiples and not), Mask words with 0 to 16 runs of kept bits
(uniform and per-position), chunk match rates from none to all, source and
slots in HBM or pinned host memory, and gathers with repeated ids.  Metadata comes from ibp_meta_create so that the
run structure and the match rate are controlled; everything the kernels
produce (stored bytes, bitmask, records, raw slots, decoded tensors, gathers)
is compared with the oracle's."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from lossless_tensor_compression_ibp_amd import ibp
from oracle import oracle
from tests.gpu_util import bitmask_bits, device, empty_like_loc, say, to_gpu

pytestmark = pytest.mark.gpu

# seeds per layout; IBP_FUZZ_CASES raises it for a longer run
N_CASES = int(os.environ.get("IBP_FUZZ_CASES", "150"))


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(force=False)


def _mask_word(rng, kind: str) -> int:
    if kind == "none":
        return 0
    if kind == "all":
        return 0xFFFFFFFF
    if kind == "high":       # sign and exponent-like: one run of kept bits
        return (0xFFFFFFFF << int(rng.integers(20, 32))) & 0xFFFFFFFF
    if kind == "dense":      # random bits: up to 16 runs of kept bits
        return int(rng.integers(0, 2**32))
    runs = int(rng.integers(1, 6))  # a few masked runs
    m = 0
    for _ in range(runs):
        a = int(rng.integers(0, 32))
        b = min(32, a + int(rng.integers(1, 6)))
        m |= ((1 << (b - a)) - 1) << a
    return m


def _format(rng, layout):
    """Chunk width, chunks per tensor and period (in chunks).  The packed
    and header-in-GPU-memory layouts take 16-byte aligned tensors of one tile
    (headers in GPU memory: at most 128 chunks) with tables in LDS."""
    W = int(rng.choice([32, 64, 128, 256, 512, 1024]))
    g = W // 32
    if layout is None:
        shape = rng.choice(["small", "small", "small", "multi"])
        if shape == "multi":
            # up to 4 tiles (one group of the decode), or up to 26 (four groups)
            top = 9000 if rng.random() < 0.5 else 53000
            n_chunks = int(rng.integers(2049 // g + 1, top // g + 2))
        else:
            n_chunks = int(rng.integers(1, max(2, 2048 // g) + 1))
        max_m = 1 << 20
    else:
        step = max(1, 4 // g)  # whole 16-byte vectors
        top = min(2048 // g, 128 if layout == "split" else 2048 // g)
        n_chunks = step * int(rng.integers(1, top // step + 1))
        max_m = 8192
    divisors = [d for d in range(1, n_chunks + 1) if n_chunks % d == 0 and d * W <= max_m]
    if not divisors:
        divisors = [1]
    d = int(rng.choice(divisors[:12] + divisors[-3:]))
    return W, n_chunks, d


def make_case(seed: int, layout: str | None = None):
    """A random format and n tensors whose chunks match at a chosen rate."""
    rng = np.random.default_rng((10_000 if layout is None else 20_000 if layout == "packed" else 30_000) + seed)
    W, n_chunks, d = _format(rng, layout)
    g = W // 32
    n_words = n_chunks * g
    L = 4 * n_words
    M = d * W
    Mw = M // 32
    kind = str(rng.choice(["none", "all", "high", "dense", "few", "mixed", "uniform"]))
    if kind == "uniform":
        w0 = _mask_word(rng, str(rng.choice(["high", "dense", "few"])))
        mask = np.full(Mw, w0, np.uint32)
    elif kind == "mixed":
        mask = np.array([_mask_word(rng, str(rng.choice(["none", "all", "high", "dense", "few"])))
                         for _ in range(Mw)], np.uint32)
    else:
        mask = np.array([_mask_word(rng, kind) for _ in range(Mw)], np.uint32)
    bitval = (rng.integers(0, 2**32, size=Mw, dtype=np.uint64).astype(np.uint32)) & mask
    if kind == "uniform":
        bitval[:] = bitval[0]
    n = int(max(1, min(300, 600_000 // L + 1)))
    q = float(rng.choice([0.0, 0.5, 0.9, 0.99, 1.0]))
    x = rng.integers(0, 2**32, size=(n, n_words), dtype=np.uint64).astype(np.uint32)
    mfull = np.tile(mask, n_words // Mw)
    bfull = np.tile(bitval, n_words // Mw)
    x = (x & ~mfull) | bfull  # every chunk matches ...
    # ... except these, which get one masked bit flipped (a chunk with no
    # masked bit matches whatever it holds); the flipped bit is drawn once per
    # chunk position
    flip_word = np.full(n_chunks, -1, np.int64)
    flip_bit = np.zeros(n_chunks, np.uint32)
    for ch in range(n_chunks):
        words = mfull[ch * g:(ch + 1) * g]
        nz = np.flatnonzero(words)
        if nz.size:
            j = int(nz[rng.integers(nz.size)])
            bits = np.flatnonzero((int(words[j]) >> np.arange(32)) & 1)
            flip_word[ch] = ch * g + j
            flip_bit[ch] = np.uint32(1 << int(bits[rng.integers(bits.size)]))
    miss = (rng.random((n, n_chunks)) >= q) & (flip_word >= 0)[None, :]
    tt, cc = np.nonzero(miss)
    x[tt, flip_word[cc]] ^= flip_bit[cc]
    raw = x.view(np.uint8).reshape(n, L)
    pinned = bool(rng.random() < 0.3)
    ids = rng.integers(0, n, size=int(rng.integers(1, 2 * n + 2)))
    # the encode's source in pinned host memory (look-back per tile) or in HBM
    # (a first pass over groups of tiles for long tensors)
    src_pinned = bool(rng.random() < 0.3)
    return dict(W=W, M=M, L=L, n=n, mask=mask, bitval=bitval, raw=raw, pinned=pinned, ids=ids, kind=kind, q=q,
                src_pinned=src_pinned)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_format(seed):
    c = make_case(seed)
    W, M, L, n, raw = c["W"], c["M"], c["L"], c["n"], c["raw"]
    say(f"[fuzz] seed={seed} W={W} M={M} L={L} n={n} mask={c['kind']} q={c['q']} pinned={c['pinned']} "
        f"src_pinned={c['src_pinned']}")
    dev = device()
    meta = ibp.ibp_meta_create(L, W, M, c["mask"], c["bitval"])
    mb, bb = c["mask"].view(np.uint8), c["bitval"].view(np.uint8)
    src = to_gpu(raw, pinned=c["src_pinned"])
    slots = empty_like_loc((n, L), torch.uint8, c["pinned"])
    bm = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bm, stored)
    torch.cuda.synchronize()
    o_slots, o_bm, o_stored = oracle.compress(raw, L, W, M, mb, bb, n)
    np.testing.assert_array_equal(bitmask_bits(bm.cpu().numpy().view(np.uint32), n), bitmask_bits(o_bm, n),
                                  err_msg="bitmask differs")
    g_stored = stored.cpu().numpy().astype(np.uint64)
    np.testing.assert_array_equal(g_stored, o_stored, err_msg="stored bytes differ")
    g_slots = slots.cpu().numpy()
    comp = bitmask_bits(o_bm, n).astype(bool)
    for t in np.flatnonzero(comp):
        k = int(o_stored[t])
        np.testing.assert_array_equal(g_slots[t, :k], o_slots[t, :k], err_msg=f"record of slot {t} differs")
    np.testing.assert_array_equal(g_slots[~comp], raw[~comp], err_msg="raw slots differ")
    out = torch.empty((n, L), dtype=torch.uint8, device=dev)
    ibp.ibp_decompress(meta, slots, bm, n, out)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(out.cpu().numpy(), raw, err_msg="decompress differs")
    # the oracle's slots decoded on the GPU, gathered with repeated ids
    o_slots_g = to_gpu(o_slots, pinned=c["pinned"])
    o_bm_g = torch.from_numpy(o_bm.view(np.int32).copy()).to(dev)
    ids = c["ids"]
    g_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).to(dev)
    gout = torch.empty((ids.size, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress(meta, o_slots_g, n, o_bm_g, g_ids, gout)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(gout.cpu().numpy(), raw[ids], err_msg="gather of oracle slots differs")
    say(f"[fuzz] seed={seed} ok: {int(comp.sum())} of {n} compressed, runs={ibp.ibp_meta_get_info(meta)['max_runs']}")
    meta.close()


def _layout_applies(c, max_header_words=None) -> bool:
    """The packed and header-in-GPU-memory layouts take 16-byte aligned
    tensors of one tile (at most 2,048 words)."""
    if c["L"] % 16 or c["L"] // 4 > 2048:
        return False
    return max_header_words is None or oracle.header_words(c["L"], c["W"]) <= max_header_words


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_format_packed(seed):
    c = make_case(seed, "packed")
    assert _layout_applies(c)
    W, M, L, n, raw = c["W"], c["M"], c["L"], c["n"], c["raw"]
    say(f"[fuzz packed] seed={seed} W={W} M={M} L={L} n={n} mask={c['kind']} q={c['q']} pinned={c['pinned']}")
    dev = device()
    meta = ibp.ibp_meta_create(L, W, M, c["mask"], c["bitval"])
    mb, bb = c["mask"].view(np.uint8), c["bitval"].view(np.uint8)
    src = to_gpu(raw, pinned=c["pinned"])
    off = torch.full((n + 1,), -1, dtype=torch.int64, device=dev)
    ibp.ibp_packed_offsets(meta, src, n, off)
    o_buf, o_off, o_bm = oracle.compress_packed(raw, L, W, M, mb, bb, n)
    np.testing.assert_array_equal(off.cpu().numpy().astype(np.uint64), o_off, err_msg="offsets differ")
    total = int(o_off[-1])
    cap = total + 64
    buf = torch.full((cap,), 0xEE, dtype=torch.uint8, pin_memory=True) if c["pinned"] else \
        torch.full((cap,), 0xEE, dtype=torch.uint8, device=dev)
    bm = torch.zeros(max(1, (n + 31) // 32), dtype=torch.int32, device=dev)
    ibp.ibp_compress_packed(meta, src, n, off, buf, bm, capacity=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    b = buf.cpu().numpy()
    np.testing.assert_array_equal(b[:total], o_buf[:total], err_msg="packed bytes differ")
    assert (b[total:] == 0xEE).all(), "wrote past the last item"
    np.testing.assert_array_equal(bm.cpu().numpy().view(np.uint32)[: o_bm.size], o_bm, err_msg="bitmask differs")
    ids = c["ids"]
    g = torch.empty((ids.size, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_packed(meta, buf, off, n, bm, torch.from_numpy(ids).to(dev), g, buf_bytes=cap)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(g.cpu().numpy(), raw[ids], err_msg="packed gather differs")
    meta.close()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_format_split(seed):
    c = make_case(seed, "split")
    assert _layout_applies(c, max_header_words=4)
    W, M, L, n, raw = c["W"], c["M"], c["L"], c["n"], c["raw"]
    hw = oracle.header_words(L, W)
    say(f"[fuzz split] seed={seed} W={W} M={M} L={L} n={n} hw={hw} mask={c['kind']} q={c['q']} pinned={c['pinned']}")
    dev = device()
    meta = ibp.ibp_meta_create(L, W, M, c["mask"], c["bitval"])
    mb, bb = c["mask"].view(np.uint8), c["bitval"].view(np.uint8)
    src = to_gpu(raw)
    slots = torch.full((n, L), 0xEE, dtype=torch.uint8, pin_memory=True) if c["pinned"] else \
        torch.full((n, L), 0xEE, dtype=torch.uint8, device=dev)
    headers = torch.full((n, hw), -1, dtype=torch.int32, device=dev)
    bm = torch.zeros(max(1, (n + 31) // 32), dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress_split(meta, src, n, slots, headers, bm, stored)
    torch.cuda.synchronize()
    o_slots, o_hdr, o_bm, o_st = oracle.compress_split(raw, L, W, M, mb, bb, n)
    np.testing.assert_array_equal(bm.cpu().numpy().view(np.uint32)[: o_bm.size], o_bm, err_msg="bitmask differs")
    np.testing.assert_array_equal(headers.cpu().numpy().view(np.uint32), o_hdr, err_msg="header words differ")
    st = stored.cpu().numpy().astype(np.uint64)
    np.testing.assert_array_equal(st, o_st, err_msg="stored bytes differ")
    sl = slots.cpu().numpy()
    for t in range(n):
        k = int(st[t])
        np.testing.assert_array_equal(sl[t, :k], o_slots[t, :k], err_msg=f"slot {t} differs")
    ids = c["ids"]
    g = torch.empty((ids.size, L), dtype=torch.uint8, device=dev)
    ibp.ibp_gather_decompress_split(meta, slots, n, headers, bm, torch.from_numpy(ids).to(dev), g)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    np.testing.assert_array_equal(g.cpu().numpy(), raw[ids], err_msg="split gather differs")
    meta.close()
