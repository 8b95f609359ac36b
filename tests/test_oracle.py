"""Pins for the CPU oracle (runs without a GPU).

The oracle is checked against things other than itself:
  * hand-derived vectors (tests/golden/hand_vectors.txt);
  * x86 BMI2 PEXT/PDEP, a hardware bit-extract/deposit, for the removal and
    reinsertion of masked bits;
  * exhaustive enumeration of every Mask/Bitval pair and every two-chunk
    tensor at tiny chunk widths;
  * closed forms (record length, all-identical samples, all-zero rows) and
    invariants (round trip, verbatim rule, threshold boundary, monotonicity
    in T, sample-order independence, corrupt-record detection).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle as O
from tests import golden_vectors
from lossless_tensor_compression_ibp_amd import workloads as WL


@pytest.fixture(scope="module", autouse=True)
def _built():
    O.build(force=False)


def popcount32(a):
    a = np.asarray(a, dtype=np.uint64)
    return np.array([bin(int(v)).count("1") for v in a.reshape(-1)], dtype=np.int64).reshape(a.shape)


# --------------------------------------------------------------------------
# Hand-derived vectors
# --------------------------------------------------------------------------
CASES = golden_vectors.load()


@pytest.mark.parametrize("case", CASES, ids=[c["case"] for c in CASES])
def test_hand_vectors(case):
    W, M, tb = case["W"], case["M"], case["tensor_bits"]
    mask, bitval, x = case["mask"], case["bitval"], case["x"]
    rec, R = O.encode_record(x, tb, W, M, mask, bitval)
    words = rec.view(np.uint32)
    assert R == case["R"]
    if "record" in case:
        np.testing.assert_array_equal(words, case["record"])
    if "record_head" in case:
        np.testing.assert_array_equal(words[: case["record_head"].size], case["record_head"])
        np.testing.assert_array_equal(words[-case["record_last"].size:], case["record_last"])
        assert words.size == case["record_words"]
    if "one_bits" in case:
        bits = np.unpackbits(rec, bitorder="little")
        assert set(np.flatnonzero(bits).tolist()) == case["one_bits"]
    # decoding gives the tensor back
    y = O.decode_record(rec, tb, W, M, mask, bitval)
    np.testing.assert_array_equal(y.view(np.uint32), x)
    # slot decision
    if case.get("L"):
        L = case["L"]
        slots, bm, stored = O.compress(x, L, W, M, mask, bitval, 1)
        if case["slot"] == "raw":
            assert bm[0] == 0 and stored[0] == L
            np.testing.assert_array_equal(slots[0].view(np.uint32), x)
        else:
            assert bm[0] == 1 and stored[0] == 4 * words.size
            np.testing.assert_array_equal(slots[0, : 4 * words.size], rec)
        back = O.decompress(slots, bm, L, W, M, mask, bitval, 1)
        np.testing.assert_array_equal(back[0].view(np.uint32), x)


# --------------------------------------------------------------------------
# BMI2 PEXT/PDEP cross-check
# --------------------------------------------------------------------------
BMI2_SRC = r"""
#include <stdint.h>
#include <immintrin.h>
void pext_n(const uint32_t* x, const uint32_t* m, uint32_t* out, int n) {
    for (int i = 0; i < n; ++i) out[i] = _pext_u32(x[i], m[i]);
}
void pdep_n(const uint32_t* x, const uint32_t* m, uint32_t* out, int n) {
    for (int i = 0; i < n; ++i) out[i] = _pdep_u32(x[i], m[i]);
}
"""


def _has_bmi2() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " bmi2" in f.read()
    except OSError:
        return False


@pytest.fixture(scope="module")
def bmi2(tmp_path_factory):
    if not _has_bmi2():
        pytest.skip("host CPU lacks BMI2")
    d = tmp_path_factory.mktemp("bmi2")
    src = d / "bmi2.c"
    so = d / "libbmi2.so"
    src.write_text(BMI2_SRC)
    subprocess.run(["gcc", "-O2", "-mbmi2", "-fPIC", "-shared", "-o", str(so), str(src)], check=True)
    lib = ctypes.CDLL(str(so))
    p = ctypes.c_void_p

    def run(fn, x, m):
        x = np.ascontiguousarray(x, np.uint32)
        m = np.ascontiguousarray(np.broadcast_to(m, x.shape), np.uint32)
        out = np.zeros_like(x)
        getattr(lib, fn)(p(x.ctypes.data), p(m.ctypes.data), p(out.ctypes.data), ctypes.c_int(x.size))
        return out

    return run


def test_pext_pdep_against_bmi2(bmi2):
    """W = M = 32, one chunk per tensor: a matched chunk's payload is
    PEXT(x, ~mask); decoding is PDEP(payload, ~mask) | Bitval."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        m = np.uint32(rng.integers(0, 2**32))
        if trial % 6 == 0:
            m = np.uint32((0xFFFFFFFF << int(rng.integers(0, 33))) & 0xFFFFFFFF)
        b = np.uint32(rng.integers(0, 2**32)) & m
        x = rng.integers(0, 2**32, size=256, dtype=np.uint64).astype(np.uint32)
        # force about half of the chunks to match
        x[::2] = (x[::2] & ~m) | b
        xs = x.view(np.uint8).reshape(-1, 4)
        mask = np.array([m], np.uint32)
        bitval = np.array([b], np.uint32)
        recs, R = O.encode_records(xs, 32, 32, 32, mask, bitval)
        rw = recs.view(np.uint32)  # (n, 2)
        match = ((x ^ b) & m) == 0
        np.testing.assert_array_equal(rw[:, 0] & 1, match.astype(np.uint32))
        k = bin(int(m)).count("1")
        np.testing.assert_array_equal(R, np.where(match, 64 - k, 64).astype(np.uint64))
        nm = np.uint32(~m & 0xFFFFFFFF)
        pext = bmi2("pext_n", x, nm)
        np.testing.assert_array_equal(rw[match, 1], pext[match])
        np.testing.assert_array_equal(rw[~match, 1], x[~match])
        # reinsertion
        y = O.decode_records(recs, 32, 32, 32, mask, bitval).view(np.uint32).reshape(-1)
        np.testing.assert_array_equal(y, x)
        pdep = bmi2("pdep_n", rw[match, 1], nm) | b
        np.testing.assert_array_equal(pdep, x[match])


# --------------------------------------------------------------------------
# Exhaustive enumeration at tiny chunk widths
# --------------------------------------------------------------------------
def _submasks(m: int):
    s = m
    while True:
        yield s
        if s == 0:
            return
        s = (s - 1) & m


@pytest.mark.parametrize("W,periods,n_chunks", [(1, 1, 2), (2, 1, 2), (3, 1, 2), (4, 1, 2), (5, 1, 2), (6, 1, 2),
                                                (2, 2, 2), (3, 2, 2), (4, 2, 2), (7, 1, 1), (8, 1, 1)])
def test_exhaustive_tiny_chunks(W, periods, n_chunks, bmi2):
    """Every (Mask, Bitval subset of Mask) pair and every tensor of n_chunks
    chunks (two chunks up to W = 6, one chunk at W = 7 and 8: 6,561 pairs x
    256 values): round trip, header = match test, record length formula,
    verbatim rule, and matched payload = PEXT of the chunk."""
    M = W * periods
    tb = n_chunks * W
    full = (1 << W) - 1
    v = np.arange(1 << tb, dtype=np.uint64)
    nbytes = (tb + 7) // 8
    xs = np.stack([((v >> np.uint64(8 * i)) & np.uint64(0xFF)).astype(np.uint8) for i in range(nbytes)], axis=1)
    xc = [((v >> np.uint64(c * W)) & np.uint64(full)).astype(np.uint32) for c in range(n_chunks)]
    n_pairs = 0
    for mask_int in range(1 << M):
        for bv_int in _submasks(mask_int):
            n_pairs += 1
            mask = np.array([mask_int], np.uint64).view(np.uint8)[: (M + 7) // 8].copy()
            bitval = np.array([bv_int], np.uint64).view(np.uint8)[: (M + 7) // 8].copy()
            recs, R = O.encode_records(xs, tb, W, M, mask, bitval)
            rv = recs.view(np.uint64).reshape(-1)  # records fit in 64 bits here
            back = O.decode_records(recs, tb, W, M, mask, bitval)
            np.testing.assert_array_equal(back, xs)
            pad = np.uint64((1 << (32 - n_chunks)) - 1)
            assert np.all((rv >> np.uint64(n_chunks)) & pad == 0)  # header padding
            payload = rv >> np.uint64(32)
            offset = np.zeros_like(v)
            expect_R = np.full(v.shape, 32, np.uint64)
            for c in range(n_chunks):
                mc = (mask_int >> ((c * W) % M)) & full
                bc = (bv_int >> ((c * W) % M)) & full
                k = bin(mc).count("1")
                match = ((xc[c] ^ np.uint32(bc)) & np.uint32(mc)) == 0
                p = ((rv >> np.uint64(c)) & np.uint64(1)).astype(bool)
                np.testing.assert_array_equal(p, match)
                size = np.where(match, W - k, W).astype(np.uint64)
                field = (payload >> offset) & ((np.uint64(1) << size) - np.uint64(1))
                np.testing.assert_array_equal(field[~match], xc[c][~match])
                ext = bmi2("pext_n", xc[c], np.uint32(~mc & full))
                np.testing.assert_array_equal(field[match], ext[match])
                offset += size
                expect_R += size
            np.testing.assert_array_equal(R, expect_R)
    assert n_pairs == 3 ** M


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------
def _random_meta(rng, M, density=0.4):
    mbits = rng.random(M) < density
    vbits = (rng.random(M) < 0.5) & mbits
    return np.packbits(mbits, bitorder="little"), np.packbits(vbits, bitorder="little")


@pytest.mark.parametrize("W,M,L", [(32, 32, 64), (32, 512, 64), (64, 256, 96), (128, 1024, 128),
                                   (1024, 8192, 1024), (8, 16, 6), (96, 192, 48)])
def test_round_trip_and_length_formula(W, M, L):
    rng = np.random.default_rng(W * 7 + M)
    mask, bitval = _random_meta(rng, M)
    n_t = 40
    tb = 8 * L
    xs = rng.integers(0, 256, size=(n_t, L), dtype=np.uint8)
    # make half of the tensors match everywhere
    mb = np.unpackbits(mask, bitorder="little")[:M].astype(bool)
    vb = np.unpackbits(bitval, bitorder="little")[:M].astype(bool)
    for t in range(0, n_t, 2):
        bits = np.unpackbits(xs[t], bitorder="little").astype(bool).reshape(-1, M)
        bits[:, mb] = vb[mb]
        xs[t] = np.packbits(bits.reshape(-1), bitorder="little")
    n = tb // W
    H = 32 * ((n + 31) // 32)
    kc = [int(np.unpackbits(mask, bitorder="little")[(c * W) % M:(c * W) % M + W].sum()) for c in range(n)]
    for t in range(n_t):
        rec, R = O.encode_record(xs[t], tb, W, M, mask, bitval)
        bits = np.unpackbits(rec, bitorder="little")
        p = bits[:n]
        assert not bits[n:H].any()
        assert R == H + n * W - sum(k * int(pc) for k, pc in zip(kc, p))
        assert not bits[R:].any()  # zero padding up to 32
        assert O.record_bits(rec, tb, W, M, mask) == R
        np.testing.assert_array_equal(O.decode_record(rec, tb, W, M, mask, bitval), xs[t])
        if t % 2 == 0:
            assert p.all()
    slots, bm, stored = O.compress(xs, L, W, M, mask, bitval, n_t)
    back = O.decompress(slots, bm, L, W, M, mask, bitval, n_t)
    np.testing.assert_array_equal(back, xs)
    for t in range(n_t):
        comp = (bm[t // 32] >> (t % 32)) & 1
        assert comp == (stored[t] < L)


def test_identical_sample_gives_full_mask_and_header_only_record():
    rng = np.random.default_rng(5)
    L, W = 256, 32
    M = 8 * L
    x = rng.integers(0, 256, size=L, dtype=np.uint8)
    sample = np.tile(x, 7)
    mask, bitval = O.build_metadata(sample, 8 * L, W, M, 0.95, 7)
    assert np.all(mask == 0xFF)
    np.testing.assert_array_equal(bitval, x)
    rec, R = O.encode_record(x, 8 * L, W, M, mask, bitval)
    n = 8 * L // W
    assert R == 32 * ((n + 31) // 32)
    np.testing.assert_array_equal(rec.view(np.uint32), np.array([0xFFFFFFFF, 0xFFFFFFFF], np.uint32))


def test_threshold_boundary():
    """K = ceil(T * n_obs): 0.95 * 1024 = 972.8 -> 973; 0.9 * 1024 = 921.6 -> 922.
    A position with exactly K agreeing observations is invariant, with K-1
    it is not; the majority value goes to Bitval."""
    n = 1024
    words = np.zeros(n, np.uint32)
    counts_one = {0: 973, 1: 972, 2: 1024 - 973, 3: 1024 - 972, 4: 922, 5: 921}
    for bit, c in counts_one.items():
        words[:c] |= np.uint32(1 << bit)
    rng = np.random.default_rng(3)
    rng.shuffle(words)
    mask, bitval = O.build_metadata(words, 32, 32, 32, 0.95, n)
    m = int(mask.view(np.uint32)[0])
    b = int(bitval.view(np.uint32)[0])
    assert (m >> 0) & 1 == 1 and (b >> 0) & 1 == 1
    assert (m >> 1) & 1 == 0 and (b >> 1) & 1 == 0
    assert (m >> 2) & 1 == 1 and (b >> 2) & 1 == 0
    assert (m >> 3) & 1 == 0
    assert (m >> 4) & 1 == 0 and (m >> 5) & 1 == 0  # 922 < 973
    assert m >> 6 == (0xFFFFFFFF >> 6)  # untouched bits: all zero -> invariant 0
    assert b & ~m == 0
    mask9, bitval9 = O.build_metadata(words, 32, 32, 32, 0.9, n)
    m9 = int(mask9.view(np.uint32)[0])
    assert (m9 >> 4) & 1 == 1 and (m9 >> 5) & 1 == 0  # 922 agree -> in, 921 -> out
    assert (m9 >> 1) & 1 == 1  # 972 >= 922
    assert m9 & m == m  # lower T never loses an invariant position


def test_metadata_properties():
    rng = np.random.default_rng(9)
    L, W, M, n = 64, 32, 256, 300
    x = rng.integers(0, 256, size=(n, L), dtype=np.uint8)
    x[:, ::4] &= 0x0F  # plenty of near-constant bits
    x[rng.random((n, L)) < 0.02] ^= 0xFF
    ms = []
    for T in (0.6, 0.8, 0.95, 1.0):
        mask, bitval = O.build_metadata(x, 8 * L, W, M, T, n)
        assert np.all(bitval & ~mask == 0)
        ms.append(np.unpackbits(mask, bitorder="little").astype(bool))
        perm = rng.permutation(n)
        mask2, bitval2 = O.build_metadata(x[perm], 8 * L, W, M, T, n)
        np.testing.assert_array_equal(mask, mask2)
        np.testing.assert_array_equal(bitval, bitval2)
    for lo, hi in zip(ms, ms[1:]):
        assert np.all(hi <= lo)  # Mask(T1) contains Mask(T2) for T1 < T2
    # per-observation counting: M smaller than a tensor counts every block
    mask_w, _ = O.build_metadata(np.zeros(128, np.uint8), 1024, 32, 32, 0.95, 1)
    assert mask_w.view(np.uint32)[0] == 0xFFFFFFFF


def test_invalid_and_corrupt_inputs():
    z = np.zeros(64, np.uint8)
    for T in (0.5, 0.3, 1.01):
        with pytest.raises(O.OracleError) as e:
            O.build_metadata(z, 512, 32, 512, T, 1)
        assert e.value.code == O.ERR_INVALID
    with pytest.raises(O.OracleError):
        O.build_metadata(z, 512, 96, 512, 0.95, 1)  # W does not divide M
    mask = np.array([0xFFFFFFFF], np.uint32)
    bitval = np.array([0], np.uint32)
    rec, R = O.encode_record(np.zeros(4, np.uint32), 128, 32, 32, mask, bitval)
    bad = rec.copy()
    bad[0] |= 0x80  # header padding bit 7 (n = 4 chunks)
    with pytest.raises(O.OracleError) as e:
        O.record_bits(bad, 128, 32, 32, mask)
    assert e.value.code == O.ERR_CORRUPT
    # a "compressed" slot whose header implies a record as long as the slot
    L = 16
    slots = np.zeros((1, L), np.uint8)  # header 0: no chunk matched -> 32 + 128 bits
    with pytest.raises(O.OracleError) as e:
        O.decompress(slots, np.array([1], np.uint32), L, 32, 32, mask, bitval, 1)
    assert e.value.code == O.ERR_CORRUPT
    slots, bm, _ = O.compress(np.zeros((2, L), np.uint8), L, 32, 32, mask, bitval, 2)
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress(slots, 2, bm, np.array([0, 2]), L, 32, 32, mask, bitval)
    assert e.value.code == O.ERR_RANGE
    out = O.gather_decompress(slots, 2, bm, np.array([1, 1, 0]), L, 32, 32, mask, bitval)
    assert out.shape == (3, L) and not out.any()


# --------------------------------------------------------------------------
# Statistical sanity on scaled-down workloads (context, not parity)
# --------------------------------------------------------------------------
def _savings(x2d: np.ndarray, wl: WL.Workload, n_sample: int) -> float:
    raw = np.ascontiguousarray(x2d).view(np.uint8).reshape(x2d.shape[0], -1)
    L = raw.shape[1]
    mask, bitval = O.build_metadata(raw[:n_sample], 8 * L, wl.chunk_bits, wl.period_bits,
                                    wl.threshold, n_sample)
    slots, bm, stored = O.compress(raw, L, wl.chunk_bits, wl.period_bits, mask, bitval, raw.shape[0])
    back = O.decompress(slots, bm, L, wl.chunk_bits, wl.period_bits, mask, bitval, raw.shape[0])
    np.testing.assert_array_equal(back, raw)
    return 1.0 - float(stored.sum()) / raw.size


def test_workload_savings_bands():
    s1 = _savings(WL.dense_gnn(2048), WL.DENSE_GNN, 1024)
    assert 0.08 < s1 < 0.22, s1
    s2 = _savings(WL.sparse_gnn(4096), WL.SPARSE_GNN, 1024)
    assert 0.28 < s2 < 0.46, s2
    s3 = _savings(WL.dlrm(4096), WL.DLRM, 1024)
    assert 0.05 < s3 < 0.13, s3


# --------------------------------------------------------------------------
# Packed cache (FR/KO summary, "Intégration au système": a software cache of
# compressed tensors holds more of them).  Items stored back to back on
# 16-byte boundaries.
# --------------------------------------------------------------------------
def _packed_golden():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "packed_vectors.txt")
    d = {}
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                k, v = (t.strip() for t in line.split(":", 1))
                d[k] = v
    L, W, M = int(d["L"]), int(d["W"]), int(d["M"])
    mism = {}
    for tok in d["mismatch"].split():
        t, rng = tok.split(":")
        a, b = map(int, rng.split("-")) if "-" in rng else (int(rng), int(rng))
        mism[int(t)] = set(range(a, b + 1))
    n = len(d["bitmask_bits"].split())
    words = np.zeros((n, L // 4), np.uint32)
    for t in range(n):
        for i in range(L // 4):
            hi = 0x4000 if i in mism.get(t, ()) else 0x3F80
            words[t, i] = (hi << 16) | (0x1000 + i)
    return dict(L=L, W=W, M=M, mask=np.array([int(d["mask"], 16)], np.uint32),
                bitval=np.array([int(d["bitval"], 16)], np.uint32), x=words,
                offsets=np.array([int(v) for v in d["offsets"].split()], np.uint64),
                bits=np.array([int(v) for v in d["bitmask_bits"].split()]),
                record0=np.array([int(v, 16) for v in d["record0"].split()], np.uint32))


def test_packed_hand_vector():
    g = _packed_golden()
    L, W, M, n = g["L"], g["W"], g["M"], g["x"].shape[0]
    off = O.packed_offsets(g["x"], L, W, M, g["mask"], g["bitval"], n)
    np.testing.assert_array_equal(off, g["offsets"])
    buf, off2, bm = O.compress_packed(g["x"], L, W, M, g["mask"], g["bitval"], n, capacity=int(off[-1]))
    np.testing.assert_array_equal(off2, g["offsets"])
    bits = (bm[0] >> np.arange(n)) & 1
    np.testing.assert_array_equal(bits, g["bits"])
    rec0 = buf[: 4 * g["record0"].size].view(np.uint32)
    np.testing.assert_array_equal(rec0, g["record0"])
    assert not buf[36:48].any(), "padding after an item is zero"
    # the raw item is the tensor itself
    np.testing.assert_array_equal(buf[112:176].view(np.uint32), g["x"][2])
    out = O.gather_decompress_packed(buf, off, n, bm, [3, 2, 1, 0, 0], L, W, M, g["mask"], g["bitval"])
    np.testing.assert_array_equal(out.view(np.uint32), g["x"][[3, 2, 1, 0, 0]])


@pytest.mark.parametrize("wl", ["sparse_gnn", "dense_gnn", "dlrm"])
def test_packed_items_are_the_slot_items(wl):
    """Cross-mode invariant: item t of the packed buffer is byte for byte the
    stored prefix of slot t, the offsets advance by that prefix rounded up to
    16 bytes, and gathers round-trip."""
    w = WL.ALL[wl]
    gen = {"sparse_gnn": WL.sparse_gnn, "dense_gnn": WL.dense_gnn, "dlrm": WL.dlrm}[wl]
    raw = np.ascontiguousarray(gen(700)).view(np.uint8).reshape(700, -1)
    n, L = raw.shape
    m, b = O.build_metadata(raw, 8 * L, w.chunk_bits, w.period_bits, w.threshold, 512)
    slots, bm_s, stored = O.compress(raw, L, w.chunk_bits, w.period_bits, m, b, n)
    buf, off, bm = O.compress_packed(raw, L, w.chunk_bits, w.period_bits, m, b, n)
    np.testing.assert_array_equal(bm, bm_s)
    assert off[0] == 0
    np.testing.assert_array_equal(np.diff(off.astype(np.int64)), (stored.astype(np.int64) + 15) // 16 * 16)
    for t in range(n):
        k = int(stored[t])
        assert np.array_equal(buf[int(off[t]): int(off[t]) + k], slots[t, :k]), t
    assert off[-1] < n * L  # the cache holds more
    ids = np.random.default_rng(3).integers(0, n, 900)
    out = O.gather_decompress_packed(buf, off, n, bm, ids, L, w.chunk_bits, w.period_bits, m, b)
    np.testing.assert_array_equal(out, raw[ids])


def test_packed_edge_cases():
    g = _packed_golden()
    L, W, M, n = g["L"], g["W"], g["M"], g["x"].shape[0]
    mk, bv = g["mask"], g["bitval"]
    # empty input
    off = O.packed_offsets(np.zeros(0, np.uint8), L, W, M, mk, bv, 0)
    np.testing.assert_array_equal(off, [0])
    # capacity: exactly enough works, one byte less is a range error
    need = int(g["offsets"][-1])
    O.compress_packed(g["x"], L, W, M, mk, bv, n, capacity=need)
    with pytest.raises(O.OracleError) as e:
        O.compress_packed(g["x"], L, W, M, mk, bv, n, capacity=need - 1)
    assert e.value.code == O.ERR_RANGE
    buf, off, bm = O.compress_packed(g["x"], L, W, M, mk, bv, n, capacity=need)
    # an id past the items
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress_packed(buf, off, n, bm, [n], L, W, M, mk, bv)
    assert e.value.code == O.ERR_RANGE
    # an item cut shorter than its record (offsets of tensor 1 end early)
    bad = off.copy()
    bad[2] = bad[1] + 48  # the 52-byte record of tensor 1 no longer fits
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress_packed(buf, bad, n, bm, [1], L, W, M, mk, bv)
    assert e.value.code == O.ERR_CORRUPT
    # a raw item shorter than the tensor
    bad = off.copy()
    bad[3] = bad[2] + 48
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress_packed(buf, bad, n, bm, [2], L, W, M, mk, bv)
    assert e.value.code == O.ERR_CORRUPT


# --------------------------------------------------------------------------
# Headers in GPU memory: the slot keeps the payload, the header words live in
# a separate (GPU-resident) array.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", [c for c in CASES if c.get("L") and "record" in c], ids=lambda c: c["case"])
def test_split_hand_vectors(case):
    """The hand-derived records, cut at the header: header words to the
    array, the rest to the slot (or the raw tensor when the record is not
    shorter than the slot)."""
    W, M, L = case["W"], case["M"], case["L"]
    mask, bitval, x, rec = case["mask"], case["bitval"], case["x"], case["record"]
    hw = O.header_words(L, W)
    slots, headers, bm, stored = O.compress_split(x, L, W, M, mask, bitval, 1)
    if case["slot"] == "raw":
        assert bm[0] == 0 and stored[0] == L
        assert not headers.any()
        np.testing.assert_array_equal(slots[0].view(np.uint32), x)
    else:
        assert bm[0] == 1 and stored[0] == 4 * (rec.size - hw)
        np.testing.assert_array_equal(headers[0], rec[:hw])
        np.testing.assert_array_equal(slots[0, : 4 * (rec.size - hw)].view(np.uint32), rec[hw:])
        assert not slots[0, 4 * (rec.size - hw):].any()
    back = O.gather_decompress_split(slots, 1, headers, bm, [0, 0], L, W, M, mask, bitval)
    np.testing.assert_array_equal(back.view(np.uint32).reshape(2, -1), np.stack([x, x]))


@pytest.mark.parametrize("wl", ["sparse_gnn", "dense_gnn", "dlrm"])
def test_split_is_the_slot_record_cut_at_the_header(wl):
    w = WL.ALL[wl]
    gen = {"sparse_gnn": WL.sparse_gnn, "dense_gnn": WL.dense_gnn, "dlrm": WL.dlrm}[wl]
    raw = np.ascontiguousarray(gen(600)).view(np.uint8).reshape(600, -1)
    n, L = raw.shape
    hw = O.header_words(L, w.chunk_bits)
    m, b = O.build_metadata(raw, 8 * L, w.chunk_bits, w.period_bits, w.threshold, 512)
    slots, bm, stored = O.compress(raw, L, w.chunk_bits, w.period_bits, m, b, n)
    s2, hdr, bm2, st2 = O.compress_split(raw, L, w.chunk_bits, w.period_bits, m, b, n)
    np.testing.assert_array_equal(bm2, bm)
    comp = ((bm[np.arange(n) >> 5] >> (np.arange(n) & 31)) & 1).astype(bool)
    np.testing.assert_array_equal(st2[comp], stored[comp] - 4 * hw)
    np.testing.assert_array_equal(st2[~comp], stored[~comp])
    for t in range(n):
        k = int(stored[t])
        if comp[t]:
            np.testing.assert_array_equal(hdr[t], slots[t, : 4 * hw].view(np.uint32))
            assert np.array_equal(s2[t, : k - 4 * hw], slots[t, 4 * hw: k]), t
        else:
            assert not hdr[t].any() and np.array_equal(s2[t], slots[t]), t
    ids = np.random.default_rng(4).integers(0, n, 800)
    out = O.gather_decompress_split(s2, n, hdr, bm2, ids, L, w.chunk_bits, w.period_bits, m, b)
    np.testing.assert_array_equal(out, raw[ids])


def test_split_errors():
    w = WL.DENSE_GNN
    raw = np.ascontiguousarray(WL.dense_gnn(64)).view(np.uint8).reshape(64, -1)
    n, L = raw.shape
    m, b = O.build_metadata(raw, 8 * L, w.chunk_bits, w.period_bits, w.threshold, 64)
    s2, hdr, bm, _ = O.compress_split(raw, L, w.chunk_bits, w.period_bits, m, b, n)
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress_split(s2, n, hdr, bm, [n], L, w.chunk_bits, w.period_bits, m, b)
    assert e.value.code == O.ERR_RANGE
    t = int(np.nonzero((bm[np.arange(n) >> 5] >> (np.arange(n) & 31)) & 1)[0][0])
    bad = hdr.copy()
    bad[t, -1] |= np.uint32(1 << 31) if (8 * L // w.chunk_bits) % 32 else 0
    if (8 * L // w.chunk_bits) % 32 == 0:
        bad[t, :] = 0  # every chunk verbatim: the record would not be shorter than the slot
    with pytest.raises(O.OracleError) as e:
        O.gather_decompress_split(s2, n, bad, bm, [t], L, w.chunk_bits, w.period_bits, m, b)
    assert e.value.code == O.ERR_CORRUPT
