"""IBP decode benchmark on one MI355X.

Default workload: sparse GNN features, 1,048,576 rows x 256 fp32 (97 % exact
zeros), chunk = 32 words (W = 1024), Mask/Bitval over the whole row
(M = 8192 bits) from the first 1,024 rows at T = 0.95.  The rows are
compressed once into fixed 1 KiB slots in pinned host memory; each step
gathers one batch of 8,192 distinct random row ids, decoding on the GPU
straight from host memory (zero copy over the host link) into HBM.

One JSON line on stdout: decoded GB/s of uncompressed output (the metric),
space savings, the roofline of the decode kernel, the host-link ceiling
measured in the same run, and the CPU oracle timed on a bounded sample.
Other workloads: --workload dense_gnn | dlrm | llm_bf16 | kv_bf16.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from lossless_tensor_compression_ibp_amd import ibp  # noqa: E402
from lossless_tensor_compression_ibp_amd import workloads as WL  # noqa: E402

GB = 1e9
PCIE5_X16_GBPS = 64.0   # PCIe 5.0 x16, one direction (MI355X host link)
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def kernel_source_hash() -> str:
    """Hash of the kernel sources; counter readings in profiles/traffic.json
    apply only while it matches."""
    import glob
    import hashlib

    csrc = os.path.join(ROOT, "lossless_tensor_compression_ibp_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp")))
    files.append(os.path.join(ROOT, "include", "ibp.h"))
    h = hashlib.sha256()
    for f in sorted(files, key=os.path.basename):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_NOTE_LINK = ("bytes per launch from rocprofv3 FETCH_SIZE (host reads over the link plus the few HBM "
                     "reads of ids and bitmask) and WRITE_SIZE (decoded rows into HBM), each scaled by what the "
                     "counter reads for a copy of known size with the same access pattern; zero-copy reads move "
                     "whole 128-byte lines")


def measured_traffic(workload: str | None):
    """Bytes per launch of the workload's decode kernel from the committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what it
    reads for a copy kernel of known size), or None when the kernels changed
    since the counters were taken."""
    if workload is None:
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    entry = t.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("traffic_bytes_per_launch")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def pinned(shape, dtype):
    return torch.empty(shape, dtype=dtype, pin_memory=True)


def h2d_ceiling(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """hipMemcpy H2D from pinned memory (GB/s, median of reps)."""
    src = pinned((nbytes,), torch.uint8)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    times = []
    for _ in range(reps + 1):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src, non_blocking=True)
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) / 1e3)
    del src, dst
    return nbytes / float(np.median(times[1:])) / GB


def copy_kernel_ceiling(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """A plain elementwise kernel (uint8 bitwise_not: reads nbytes, writes
    nbytes) as the HBM reference: GB/s of read + write traffic, median."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    times = []
    for _ in range(reps + 1):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        torch.bitwise_not(a, out=b)
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) / 1e3)
    del a, b
    return 2 * nbytes / float(np.median(times[1:])) / GB


def timed(fn, steps: int, warmup: int):
    """Runs fn(i) warmup times, then times exactly `steps` calls between two
    synchronisations.  Returns (wall seconds, launch durations in seconds):
    one HIP event pair on the launching stream brackets the whole timed
    region, and each launch is credited the region's GPU time / steps (events
    around every launch would put their own gaps between the kernels)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.full(steps, start.elapsed_time(end) / 1e3 / steps)


def encode_seconds(fn, reps: int = 3) -> float:
    """Median wall time of `reps` synchronised calls after one untimed call."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def queued_durations(fn, steps: int, first: int = 0):
    """Average launch duration of `steps` calls queued behind a bounded spin
    kernel so that the GPU runs them back to back (one event pair over the
    whole region, divided by the launches): for launches shorter than the
    host's submission time, events around each launch would also measure the
    idle gap before it."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(50_000_000)
    start.record(stream)
    for i in range(steps):
        fn(first + i)
    end.record(stream)
    torch.cuda.synchronize()
    return np.full(steps, start.elapsed_time(end) / 1e3 / steps)


def cpu_oracle_gather(raw_rows: np.ndarray, w: WL.Workload, batch: int, budget_s: float,
                      sample_rows: int) -> dict:
    """The oracle, single-threaded, decoding random batches of rows (headers
    in a separate array, as the GPU line does) from its own slots until the
    time budget is spent (encode excluded)."""
    from oracle import oracle

    oracle.build(force=False)
    sub = np.ascontiguousarray(raw_rows[:sample_rows])
    L = sub.shape[1]
    mask, bitval = oracle.build_metadata(sub[: w.n_sample], 8 * L, w.chunk_bits, w.period_bits,
                                         w.threshold, min(w.n_sample, sub.shape[0]))
    slots, headers, bm, _ = oracle.compress_split(sub, L, w.chunk_bits, w.period_bits, mask, bitval, sub.shape[0])
    rng = np.random.default_rng(WL.ID_SEED)
    rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        ids = rng.choice(sub.shape[0], batch, replace=False)
        oracle.gather_decompress_split(slots, sub.shape[0], headers, bm, ids, L, w.chunk_bits, w.period_bits,
                                       mask, bitval)
        rows += batch
    dt = time.perf_counter() - t0
    return {"value": round(rows * L / dt / GB, 6), "unit": "GB/s", "cores": 1, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{rows} rows decoded by gather in batches of {batch} ids from the oracle's slots of "
                      f"the first {sample_rows} rows ({dt:.1f} s, single thread)"}


# ---------------------------------------------------------------------------
# Sparse GNN: zero-copy gather from pinned host slots (default workload)
def cpu_oracle_roundtrip(rows: np.ndarray, w: WL.Workload, n_sample: int, budget_s: float, what: str) -> dict:
    """The oracle, single-threaded: metadata from the first n_sample rows,
    then compress and decompress of all the rows, repeated until the time
    budget is spent.  value: GB/s of decoded tensor; encode_GBps beside it."""
    from oracle import oracle

    oracle.build(force=False)
    rows = np.ascontiguousarray(rows)
    n, L = rows.shape
    mask, bitval = oracle.build_metadata(rows[:n_sample], 8 * L, w.chunk_bits, w.period_bits, w.threshold,
                                         n_sample)
    t_enc = t_dec = 0.0
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        a = time.perf_counter()
        slots, bm, _ = oracle.compress(rows, L, w.chunk_bits, w.period_bits, mask, bitval, n)
        b = time.perf_counter()
        out = oracle.decompress(slots, bm, L, w.chunk_bits, w.period_bits, mask, bitval, n)
        t_enc += b - a
        t_dec += time.perf_counter() - b
        reps += 1
    if not np.array_equal(out, rows):
        raise SystemExit("oracle round trip differs")
    return {"value": round(reps * n * L / t_dec / GB, 6), "unit": "GB/s", "cores": 1, "host_cores": os.cpu_count(),
            "kind": "oracle", "encode_GBps": round(reps * n * L / t_enc / GB, 6),
            "sample": f"{what}: {reps} compress + decompress round trips ({t_enc + t_dec:.1f} s, single thread)"}


def cpu_oracle_gather_slots(rows: np.ndarray, w: WL.Workload, batch: int, budget_s: float, what: str,
                            packed: bool = False, replace: bool = True) -> dict:
    """The oracle, single-threaded, decoding random id batches from its own
    slots (or packed items) of the sampled rows until the time budget is
    spent (encode excluded)."""
    from oracle import oracle

    oracle.build(force=False)
    rows = np.ascontiguousarray(rows)
    n, L = rows.shape
    ns = min(w.n_sample, n)
    mask, bitval = oracle.build_metadata(rows[:ns], 8 * L, w.chunk_bits, w.period_bits, w.threshold, ns)
    if packed:
        buf, off, bm = oracle.compress_packed(rows, L, w.chunk_bits, w.period_bits, mask, bitval, n)
    else:
        slots, bm, _ = oracle.compress(rows, L, w.chunk_bits, w.period_bits, mask, bitval, n)
    rng = np.random.default_rng(WL.ID_SEED)
    done = 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        ids = rng.choice(n, batch, replace=replace)
        if packed:
            oracle.gather_decompress_packed(buf, off, n, bm, ids, L, w.chunk_bits, w.period_bits, mask, bitval)
        else:
            oracle.gather_decompress(slots, n, bm, ids, L, w.chunk_bits, w.period_bits, mask, bitval)
        done += batch
    dt = time.perf_counter() - t0
    return {"value": round(done * L / dt / GB, 6), "unit": "GB/s", "cores": 1, "host_cores": os.cpu_count(),
            "kind": "oracle", "sample": f"{done} rows decoded by gather in batches of {batch} ids from the oracle's "
                                        f"{'packed items' if packed else 'slots'} of {what} ({dt:.1f} s, single thread)"}


# ---------------------------------------------------------------------------
def run_sparse_gnn(args) -> dict:
    """Zero-copy gathers of 8,192 random rows from pinned host slots.  The
    timed layout keeps each compressed row's header word in HBM beside the
    bitmask, so the host link carries payload only (a row of j non-zero
    chunks costs j lines of 128 bytes instead of j + 1); the plain slot layout
    (header in the slot) and the uncompressed rows are timed in the same run."""
    w = WL.SPARSE_GNN
    n, L = w.n_tensors if not args.small else 65536, w.tensor_bytes
    batch = 8192
    log(f"[bench] sparse_gnn: generating {n} x 256 fp32 rows")
    host = pinned((n, L), torch.uint8)
    WL.sparse_gnn(n, out=host.numpy().view(np.float32).reshape(n, 256))
    raw_np = host.numpy()
    dev = torch.device("cuda")

    log("[bench] metadata from the first 1,024 rows (zero copy from pinned memory)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    meta = ibp.ibp_build_metadata(host, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    t_meta = time.perf_counter() - t0
    info = ibp.ibp_meta_get_info(meta)
    hw = ibp.header_words(meta)

    log("[bench] compress all rows into pinned host slots, headers in HBM (zero copy both ways)")
    slots = pinned((n, L), torch.uint8)
    headers = torch.zeros((n, hw), dtype=torch.int32, device=dev)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    enc_s = []
    for _ in range(4):
        t0 = time.perf_counter()
        ibp.ibp_compress_split(meta, host, n, slots, headers, bitmask, stored)
        torch.cuda.synchronize()
        enc_s.append(time.perf_counter() - t0)
    payload_np = stored.cpu().numpy()
    comp_np = (bitmask.cpu().numpy().view(np.uint32)[np.arange(n) >> 5] >> (np.arange(n) & 31)) & 1
    # compressed bytes: payload in the slots plus the header words kept in HBM
    savings = 1.0 - (payload_np.sum() + 4 * hw * comp_np.sum()) / (n * L)

    log("[bench] the plain slot layout (header in the slot) for comparison")
    slots_plain = pinned((n, L), torch.uint8)
    bitmask_plain = torch.zeros_like(bitmask)
    stored_plain = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress(meta, host, n, slots_plain, bitmask_plain, stored_plain)
    torch.cuda.synchronize()
    stored_plain_np = stored_plain.cpu().numpy()

    ids_all = WL.batch_ids(n, batch, args.warmup + args.steps, replace=False)
    ids_dev = torch.from_numpy(ids_all).to(dev)
    out = torch.empty((2, batch, L), dtype=torch.uint8, device=dev)
    last = args.warmup + args.steps - 1

    def step(i):
        ibp.ibp_gather_decompress_split(meta, slots, n, headers, bitmask, ids_dev[i], out[i & 1])

    log(f"[bench] timing {args.steps} gather steps of {batch} rows (warmup {args.warmup})")
    wall, durs = timed(step, args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not np.array_equal(out[last & 1].cpu().numpy(), raw_np[ids_all[last]]):
        raise SystemExit("decoded rows differ from the source rows")
    timed_ids = ids_all[args.warmup:]
    link_bytes = payload_np[timed_ids].sum(axis=1)        # bytes read over the link per launch
    out_bytes = batch * L
    value = args.steps * out_bytes / wall / GB

    def plain_step(i):
        ibp.ibp_gather_decompress(meta, slots_plain, n, bitmask_plain, ids_dev[i], out[i & 1])

    plain_wall, plain_durs = timed(plain_step, args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not np.array_equal(out[last & 1].cpu().numpy(), raw_np[ids_all[last]]):
        raise SystemExit("decoded rows (slot layout) differ from the source rows")

    # raw zero-copy gather of the same rows (every bitmask bit 0): the
    # uncompressed transfer the codec competes with
    zero_bm = torch.zeros_like(bitmask)

    def raw_step(i):
        ibp.ibp_gather_decompress(meta, host, n, zero_bm, ids_dev[i], out[i & 1])

    if args.no_raw:
        raw_wall = float("nan")
    else:
        raw_wall, _ = timed(raw_step, args.steps, args.warmup)
    h2d = h2d_ceiling()
    achieved = float(link_bytes.mean() / durs.mean() / GB)
    comp_fraction = 1.0 - savings
    res = {
        "metric": "IBP decode GB/s (uncompressed out, 1 MI355X) + % of roofline + space savings %",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": f"sparse_gnn: {n} rows x 256 fp32 (97% zeros), W=1024, M=8192, T=0.95, "
                               f"1 KiB slots in pinned host memory (payload only; each compressed row's header "
                               f"word in HBM beside the bitmask), zero-copy gather of {batch} distinct random "
                               f"row ids per step into HBM",
                   "rows": n, "tensor_bytes": L, "batch_ids": batch, "chunk_bits": w.chunk_bits,
                   "period_bits": w.period_bits, "threshold": w.threshold, "layout": "headers in HBM",
                   "hbm_header_bytes": int(4 * hw * n), "hbm_bitmask_bytes": int(4 * ((n + 31) // 32))},
        "space_savings_pct": round(100 * savings, 3),
        "kernel": "ibp::k_decode_small<0, true, true, 1, true>",
        "kernel_avg_us": round(float(durs.mean()) * 1e6, 2),
        "roofline": {
            "bound": "pcie",
            "achieved": round(achieved, 3),
            "peak": PCIE5_X16_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PCIE5_X16_GBPS, 4),
            "traffic": None if args.small else measured_traffic("sparse_gnn"),
            "traffic_note": TRAFFIC_NOTE_LINK,
            "link_ceiling_measured": round(h2d, 3),
            "frac_of_measured_ceiling": round(achieved / h2d, 4),
            "algorithmic_bytes_per_launch": int(link_bytes.mean()),
        },
        # decoded throughput against link bandwidth / compressed fraction
        "decoded_roofline_GBps": round(h2d / comp_fraction, 3),
        "decoded_frac_of_roofline": round(value / (h2d / comp_fraction), 4),
        "decoded_frac_of_published_link_roofline": round(value / (PCIE5_X16_GBPS / comp_fraction), 4),
        "slot_layout": {"decoded_GBps": round(args.steps * out_bytes / plain_wall / GB, 3),
                        "kernel_avg_us": round(float(plain_durs.mean()) * 1e6, 2),
                        "link_bytes_per_launch": int(stored_plain_np[timed_ids].sum(axis=1).mean())},
        "raw_zero_copy_gather_GBps": round(args.steps * out_bytes / raw_wall / GB, 3),
        "speedup_vs_raw_zero_copy": round(raw_wall / wall, 3),
        "encode_GBps": round(n * L / float(np.median(enc_s[1:])) / GB, 3),
        "metadata_ms": round(t_meta * 1e3, 2),
        "meta": info,
    }
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_oracle_gather(raw_np, w, batch=1024, budget_s=args.cpu_budget,
                                                sample_rows=16384)
    return res


# ---------------------------------------------------------------------------
# KV cache: HBM-resident pages, compress on device, decode every page
# ---------------------------------------------------------------------------
def run_kv_bf16(args) -> dict:
    w = WL.KV_BF16
    layers = 32 if not args.small else 4
    log(f"[bench] kv_bf16: generating {layers} layers x 32 heads x 4096 tokens x 128 bf16")
    kv = WL.kv_cache(n_layers=layers)
    raw_np = kv.reshape(-1, 2048).view(np.uint8).reshape(-1, 4096)
    n, L = raw_np.shape
    dev = torch.device("cuda")
    src = torch.from_numpy(raw_np).to(dev)
    del kv, raw_np
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    meta = ibp.ibp_build_metadata(src, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    t_meta = time.perf_counter() - t0
    slots = torch.empty_like(src)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    _, enc_durs = timed(lambda i: ibp.ibp_compress(meta, src, n, slots, bitmask, stored), 5, 1)
    stored_np = stored.cpu().numpy()
    savings = 1.0 - stored_np.sum() / (n * L)
    out = torch.empty_like(src)
    wall, durs = timed(lambda i: ibp.ibp_decompress(meta, slots, bitmask, n, out), args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not torch.equal(out, src):
        raise SystemExit("decoded pages differ")
    hbm_bytes = float(stored_np.sum() + n * L + 4 * ((n + 31) // 32))
    roof = hbm_roofline(hbm_bytes, durs, None if args.small else "kv_bf16")
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_oracle_roundtrip(src[:2048].cpu().numpy(), w, w.n_sample, args.cpu_budget,
                                   "the first 2,048 pages (8 MiB; metadata from their first 1,024)")
    res = base_result(
        args, n * L * args.steps / wall / GB, wall,
        {"workload": f"kv_bf16: {layers} layers x 32 heads x 4096 tokens x 128 bf16, 4 KiB pages in HBM slots, "
                     f"W=32, M=32768, T=0.95, decode of all {n} pages per step", "pages": n, "tensor_bytes": L},
        savings, "ibp::k_decode_small<3, false, true, 4, false>", durs, roof,
        encode_GBps=round(n * L / float(np.mean(enc_durs)) / GB, 3), metadata_ms=round(t_meta * 1e3, 2),
        meta=ibp.ibp_meta_get_info(meta))
    if cpu:
        res["cpu_baseline"] = cpu
    return res


METRIC = "IBP decode GB/s (uncompressed out, 1 MI355X) + % of roofline + space savings %"


def base_result(args, value, wall, config, savings, kernel, durs, roofline, **extra) -> dict:
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": config, "space_savings_pct": round(100 * savings, 3), "kernel": kernel,
        "kernel_avg_us": round(float(np.mean(durs)) * 1e6, 2), "roofline": roofline,
    }
    res.update(extra)
    return res


def hbm_roofline(bytes_per_launch: float, durs, workload: str) -> dict:
    achieved = bytes_per_launch / float(np.mean(durs)) / GB
    return {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(workload),
            "copy_kernel_ceiling_measured": round(copy_kernel_ceiling(), 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch)}


def link_roofline(link_bytes_per_launch: float, durs, savings: float, workload: str) -> dict:
    achieved = link_bytes_per_launch / float(np.mean(durs)) / GB
    h2d = h2d_ceiling()
    return {"bound": "pcie", "achieved": round(achieved, 3), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
            "frac": round(achieved / PCIE5_X16_GBPS, 4), "traffic": measured_traffic(workload),
            "traffic_note": TRAFFIC_NOTE_LINK,
            "link_ceiling_measured": round(h2d, 3), "frac_of_measured_ceiling": round(achieved / h2d, 4),
            "algorithmic_bytes_per_launch": int(link_bytes_per_launch),
            "decoded_roofline_GBps": round(h2d / (1.0 - savings), 3)}


# ---------------------------------------------------------------------------
# Dense GNN: 8 MiB of rows in HBM, contiguous decode of the whole table
# ---------------------------------------------------------------------------
def run_dense_gnn(args) -> dict:
    w = WL.DENSE_GNN
    x = WL.dense_gnn()
    raw_np = np.ascontiguousarray(x).view(np.uint8).reshape(x.shape[0], -1)
    n, L = raw_np.shape
    dev = torch.device("cuda")
    src = torch.from_numpy(raw_np).to(dev)
    meta = ibp.ibp_build_metadata(src, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = torch.empty_like(src)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    _, enc_durs = timed(lambda i: ibp.ibp_compress(meta, src, n, slots, bitmask, stored), 20, 2)
    stored_np = stored.cpu().numpy()
    savings = 1.0 - stored_np.sum() / (n * L)
    out = torch.empty_like(src)
    wall, _ = timed(lambda i: ibp.ibp_decompress(meta, slots, bitmask, n, out), args.steps, args.warmup)
    # launches shorter than their host submission: time them queued back to back
    durs = queued_durations(lambda i: ibp.ibp_decompress(meta, slots, bitmask, n, out), args.steps)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not torch.equal(out, src):
        raise SystemExit("decoded rows differ")
    hbm_bytes = float(stored_np.sum() + n * L + 4 * ((n + 31) // 32))
    # the same rows held uncompressed: a plain device copy of them, timed the
    # same two ways (the floor of any pass over this many bytes at this size)
    raw_copy = torch.empty_like(src)
    raw_wall, _ = timed(lambda i: raw_copy.copy_(src), args.steps, args.warmup)
    raw_durs = queued_durations(lambda i: raw_copy.copy_(src), args.steps)
    del raw_copy
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_oracle_roundtrip(src.cpu().numpy(), w, w.n_sample, args.cpu_budget,
                                   f"all {n} rows (8 MiB; metadata from the first 1,024)")
    res = base_result(
        args, n * L * args.steps / wall / GB, wall,
        {"workload": f"dense_gnn: {n} rows x 128 fp32 |N(0,0.5)| with 3% N(0,50) rows, W=32, M=4096, T=0.95, "
                     f"slots in HBM, contiguous decode of all rows per step", "rows": n, "tensor_bytes": L},
        savings, "ibp::k_decode_small<1, false, true, 1, false>", durs, hbm_roofline(hbm_bytes, durs, "dense_gnn"),
        encode_GBps=round(n * L / float(np.mean(enc_durs)) / GB, 3),
        uncompressed_hbm_copy_GBps=round(n * L * args.steps / raw_wall / GB, 3),
        uncompressed_copy_kernel_us=round(float(np.mean(raw_durs)) * 1e6, 2), meta=ibp.ibp_meta_get_info(meta))
    if cpu:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------------------
# DLRM: 2 GiB embedding table in pinned host slots, 26 gathers of 65,536 ids
# ---------------------------------------------------------------------------
def run_dlrm(args) -> dict:
    w = WL.DLRM
    n = w.n_tensors if not args.small else 262144
    L = w.tensor_bytes
    batch, per_step = 65536, 26
    log(f"[bench] dlrm: generating {n} x 128 fp32 rows")
    host = pinned((n, L), torch.uint8)
    WL.dlrm(n, out=host.numpy().view(np.float32).reshape(n, 128))
    raw_np = host.numpy()
    dev = torch.device("cuda")
    meta = ibp.ibp_build_metadata(host, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = pinned((n, L), torch.uint8)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    t_enc = encode_seconds(lambda: ibp.ibp_compress(meta, host, n, slots, bitmask, stored))
    stored_np = stored.cpu().numpy()
    savings = 1.0 - stored_np.sum() / (n * L)
    n_batches = per_step * (args.warmup + args.steps)
    ids_np = WL.batch_ids(n, batch, n_batches, replace=True)
    ids = torch.from_numpy(ids_np).to(dev)
    out = torch.empty((2, batch, L), dtype=torch.uint8, device=dev)
    def step(i):
        for j in range(per_step):
            k = i * per_step + j
            ibp.ibp_gather_decompress(meta, slots, n, bitmask, ids[k], out[k & 1])

    wall, step_durs = timed(step, args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    last = n_batches - 1
    if not np.array_equal(out[last & 1].cpu().numpy(), raw_np[ids_np[last]]):
        raise SystemExit("decoded rows differ")
    durs = np.full(args.steps * per_step, float(step_durs.mean()) / per_step)  # per gather launch
    link = float(stored_np[ids_np[args.warmup * per_step:]].sum(axis=1).mean())
    value = args.steps * per_step * batch * L / wall / GB
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_oracle_gather_slots(raw_np[:65536], w, 8192, args.cpu_budget, "the first 65,536 rows (32 MiB)")
    res = base_result(
        args, value, wall,
        {"workload": f"dlrm: {n} rows x 128 fp32 U(-0.01,0.01), W=32, M=4096, T=0.9, slots in pinned host "
                     f"memory, {per_step} zero-copy gathers of {batch} random ids (with replacement) per step",
         "rows": n, "tensor_bytes": L, "batch_ids": batch, "gathers_per_step": per_step},
        savings, "ibp::k_decode_small<2, true, true, 1, false>", durs,
        link_roofline(link, durs, savings, None if args.small else "dlrm"),
        encode_GBps=round(n * L / t_enc / GB, 3), meta=ibp.ibp_meta_get_info(meta))
    if cpu:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------------------
# LLM BF16 weights: 32 layers streamed from pinned host slots, one layer of
# prefetch: decode of layer i+1 (stream A) overlaps a consumer of layer i
# (stream B, y = x @ W on the decoded layer)
# ---------------------------------------------------------------------------
def run_llm_bf16(args) -> dict:
    w = WL.LLM_BF16
    layers = 32 if not args.small else 4
    rows, cols = 4096, 11008
    L = rows * cols * 2
    log(f"[bench] llm_bf16: generating {layers} layers of {rows} x {cols} bf16")
    host = pinned((layers, L), torch.uint8)
    hv = WL.llm_layers(host.numpy(), rows, cols)
    dev = torch.device("cuda")
    meta = ibp.ibp_build_metadata(host, 1, L, w.chunk_bits, w.period_bits, w.threshold)
    slots = pinned((layers, L), torch.uint8)
    bitmask = torch.zeros((layers + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(layers, dtype=torch.int64, device=dev)
    t_enc = encode_seconds(lambda: ibp.ibp_compress(meta, host, layers, slots, bitmask, stored))
    stored_np = stored.cpu().numpy()
    savings = 1.0 - stored_np.sum() / (layers * L)
    bufs = [torch.empty(L, dtype=torch.uint8, device=dev) for _ in range(2)]
    ids = torch.arange(layers, dtype=torch.int64, device=dev)
    x = torch.randn((1, rows), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, cols), dtype=torch.bfloat16, device=dev)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    evs = []

    def one_pass(record: bool):
        ready = [torch.cuda.Event() for _ in range(layers)]
        freed = [torch.cuda.Event() for _ in range(layers)]
        for l in range(layers):
            with torch.cuda.stream(sa):
                if l >= 2:
                    sa.wait_event(freed[l - 2])
                if record:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(sa)
                ibp.ibp_gather_decompress(meta, slots, layers, bitmask, ids[l:l + 1], bufs[l & 1], stream=sa)
                if record:
                    e1.record(sa)
                    evs.append((e0, e1))
                ready[l].record(sa)
            with torch.cuda.stream(sb):
                sb.wait_event(ready[l])
                torch.matmul(x, bufs[l & 1].view(torch.bfloat16).view(rows, cols), out=y)
                freed[l].record(sb)

    for _ in range(args.warmup):
        one_pass(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_pass(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not np.array_equal(bufs[(layers - 1) & 1].cpu().numpy(), hv[layers - 1]):
        raise SystemExit("decoded layer differs")
    durs = np.array([a.elapsed_time(b) / 1e3 for a, b in evs])
    link = float(stored_np.mean())
    value = args.steps * layers * L / wall / GB
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        # one tensor made of the first 256 rows of layer 0 (5.6 MB), its own sample
        cpu = cpu_oracle_roundtrip(hv[0].reshape(1, -1)[:, : 256 * cols * 2], w, 1, args.cpu_budget,
                                   "one 5.6 MB tensor: the first 256 rows of layer 0 (metadata from itself)")
    res = base_result(
        args, value, wall,
        {"workload": f"llm_bf16: {layers} layers of {rows}x{cols} bf16 N(0,0.02) (0.1% columns x20), W=32, M=32, "
                     f"T=0.95, slots in pinned host memory, each layer decoded zero-copy into HBM on one stream "
                     f"while a consumer (y = x @ W) reads the previous layer on another", "layers": layers,
         "tensor_bytes": L},
        savings, "ibp::k_decode_tiles<3, true, true> (look-back)", durs,
        link_roofline(link, durs, savings, None if args.small else "llm_bf16"),
        encode_GBps=round(layers * L / t_enc / GB, 3), meta=ibp.ibp_meta_get_info(meta))
    if cpu:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------------------
# Sparse GNN feature cache in HBM, packed layout (items back to back)
# ---------------------------------------------------------------------------
def run_sparse_gnn_cache(args) -> dict:
    w = WL.SPARSE_GNN
    n, L = w.n_tensors if not args.small else 65536, w.tensor_bytes
    batch = 8192
    dev = torch.device("cuda")
    log(f"[bench] sparse_gnn_cache: generating {n} x 256 fp32 rows")
    host = pinned((n, L), torch.uint8)
    WL.sparse_gnn(n, out=host.numpy().view(np.float32).reshape(n, 256))
    raw_np = host.numpy()
    meta = ibp.ibp_build_metadata(host, w.n_sample, L, w.chunk_bits, w.period_bits, w.threshold)

    log("[bench] cache fill: item offsets, then the packed items into HBM (zero copy from pinned memory)")
    offsets = torch.empty(n + 1, dtype=torch.int64, device=dev)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    ibp.ibp_packed_offsets(meta, host, n, offsets)
    total = int(offsets[-1].item())
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    ibp.ibp_compress_packed(meta, host, n, offsets, buf, bitmask)
    torch.cuda.synchronize()
    fill_s = []
    for _ in range(3):
        t0 = time.perf_counter()
        ibp.ibp_packed_offsets(meta, host, n, offsets)
        ibp.ibp_compress_packed(meta, host, n, offsets, buf, bitmask)
        torch.cuda.synchronize()
        fill_s.append(time.perf_counter() - t0)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    off_np = offsets.cpu().numpy()
    item_bytes = np.diff(off_np)

    ids_all = WL.batch_ids(n, batch, args.warmup + args.steps, replace=False)
    ids_dev = torch.from_numpy(ids_all).to(dev)
    out = torch.empty((2, batch, L), dtype=torch.uint8, device=dev)

    def step(i):
        ibp.ibp_gather_decompress_packed(meta, buf, offsets, n, bitmask, ids_dev[i], out[i & 1])

    log(f"[bench] timing {args.steps} gathers of {batch} rows from the packed HBM cache")
    wall, _ = timed(step, args.steps, args.warmup)
    durs = queued_durations(step, args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    last = args.warmup + args.steps - 1
    step(last)
    if not np.array_equal(out[last & 1].cpu().numpy(), raw_np[ids_all[last]]):
        raise SystemExit("decoded rows differ from the source rows")
    timed_ids = ids_all[args.warmup:]
    # algorithmic bytes per launch: items read + rows written + ids, offsets and bitmask words
    hbm_bytes = float(item_bytes[timed_ids].sum(axis=1).mean() + batch * (L + 8 + 16 + 4))

    # the same gathers from an uncompressed HBM copy of the table
    table = host.to(dev)
    raw_wall, _ = timed(lambda i: torch.index_select(table, 0, ids_dev[i], out=out[i & 1]), args.steps,
                        args.warmup)
    raw_durs = queued_durations(lambda i: torch.index_select(table, 0, ids_dev[i], out=out[i & 1]), args.steps,
                                args.warmup)
    del table
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_oracle_gather_slots(raw_np[:16384], w, 1024, args.cpu_budget, "the first 16,384 rows (16 MiB)",
                                      packed=True, replace=False)
    res = base_result(
        args, batch * L * args.steps / wall / GB, wall,
        {"workload": f"sparse_gnn_cache: {n} rows x 256 fp32 (97% zeros), W=1024, M=8192, T=0.95, all rows "
                     f"compressed into one packed HBM buffer (items back to back, 16-byte aligned), gather of "
                     f"{batch} distinct random row ids per step into HBM", "rows": n, "tensor_bytes": L,
         "batch_ids": batch},
        1.0 - total / (n * L), "ibp::k_decode_small<0, true, true, 1, false> (packed items)", durs,
        hbm_roofline(hbm_bytes, durs, None if args.small else "sparse_gnn_cache"),
        cache_bytes=total, capacity_gain=round(n * L / total, 4),
        fill_GBps=round(n * L / float(np.median(fill_s)) / GB, 3),
        uncompressed_hbm_gather_GBps=round(batch * L * args.steps / raw_wall / GB, 3),
        uncompressed_gather_kernel_us=round(float(np.mean(raw_durs)) * 1e6, 2),
        meta=ibp.ibp_meta_get_info(meta))
    if cpu:
        res["cpu_baseline"] = cpu
    return res


# ---------------------------------------------------------------------------
# Chunk width x threshold sweep (sparse rows) and an fp16 variant (dense rows)
# ---------------------------------------------------------------------------
def run_sweep(args) -> dict:
    """Savings and gather rate across chunk widths W and thresholds T on a
    262,144-row slice of the sparse_gnn table (pinned slots, plain layout,
    8,192 distinct ids per gather), and the dense_gnn rows stored as fp16.
    `value` is the point of the sparse_gnn line itself (W = 1,024, T = 0.95)."""
    w = WL.SPARSE_GNN
    n, L = (262144 if not args.small else 32768), w.tensor_bytes
    batch = 8192
    dev = torch.device("cuda")
    log(f"[bench] sweep: generating {n} x 256 fp32 sparse rows")
    host = pinned((n, L), torch.uint8)
    WL.sparse_gnn(n, out=host.numpy().view(np.float32).reshape(n, 256))
    raw_np = host.numpy()
    slots = pinned((n, L), torch.uint8)
    bitmask = torch.zeros((n + 31) // 32, dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ids_all = WL.batch_ids(n, batch, args.warmup + args.steps, replace=False)
    ids_dev = torch.from_numpy(ids_all).to(dev)
    out = torch.empty((2, batch, L), dtype=torch.uint8, device=dev)
    points, value, wall_at, durs_at = [], None, None, None
    for W in (32, 64, 128, 256, 512, 1024):
        for T in (0.9, 0.95, 0.99):
            meta = ibp.ibp_build_metadata(host, w.n_sample, L, W, w.period_bits, T)
            ibp.ibp_compress(meta, host, n, slots, bitmask, stored)
            st = stored.cpu().numpy()

            def step(i, meta=meta):
                ibp.ibp_gather_decompress(meta, slots, n, bitmask, ids_dev[i], out[i & 1])

            wall, durs = timed(step, args.steps, args.warmup)
            assert ibp.ibp_check(meta) == ibp.IBP_OK
            last = args.warmup + args.steps - 1
            if not np.array_equal(out[last & 1].cpu().numpy(), raw_np[ids_all[last]]):
                raise SystemExit(f"decoded rows differ at W={W} T={T}")
            gbps = args.steps * batch * L / wall / GB
            points.append({"W": W, "T": T, "savings_pct": round(100 * (1 - st.sum() / (n * L)), 3),
                           "decoded_GBps": round(gbps, 3), "kernel_avg_us": round(float(durs.mean()) * 1e6, 2),
                           "link_bytes_per_launch": int(st[ids_all[args.warmup:]].sum(axis=1).mean()),
                           "uniform_metadata": bool(ibp.ibp_meta_get_info(meta)["uniform"])})
            log(f"[bench] sweep W={W} T={T}: {points[-1]['savings_pct']} % saved, {gbps:.1f} GB/s decoded")
            if W == w.chunk_bits and T == w.threshold:
                value, wall_at, durs_at = gbps, wall, durs
                link_at = float(points[-1]["link_bytes_per_launch"])
                savings_at = points[-1]["savings_pct"] / 100
            meta.close()
    # dense_gnn rows as fp16: 16,384 rows x 128 half, HBM slots, all rows per step
    wd = WL.DENSE_GNN
    x16 = WL.dense_gnn().astype(np.float16)
    raw16 = np.ascontiguousarray(x16).view(np.uint8).reshape(x16.shape[0], -1)
    src16 = torch.from_numpy(raw16).to(dev)
    n16, L16 = raw16.shape
    fp16 = []
    for W in (32, 64):
        meta = ibp.ibp_build_metadata(src16, wd.n_sample, L16, W, 8 * L16, wd.threshold)
        s16 = torch.empty_like(src16)
        b16 = torch.zeros((n16 + 31) // 32, dtype=torch.int32, device=dev)
        st16 = torch.zeros(n16, dtype=torch.int64, device=dev)
        ibp.ibp_compress(meta, src16, n16, s16, b16, st16)
        o16 = torch.empty_like(src16)
        wall, _ = timed(lambda i: ibp.ibp_decompress(meta, s16, b16, n16, o16), args.steps, args.warmup)
        assert ibp.ibp_check(meta) == ibp.IBP_OK and torch.equal(o16, src16)
        fp16.append({"W": W, "T": wd.threshold, "M": 8 * L16,
                     "savings_pct": round(100 * (1 - st16.cpu().numpy().sum() / (n16 * L16)), 3),
                     "decoded_GBps": round(args.steps * n16 * L16 / wall / GB, 3)})
        meta.close()
    return base_result(
        args, value, wall_at,
        {"workload": f"sweep: sparse_gnn rows ({n} x 256 fp32, 97% zeros), M=8192, chunk widths W=32..1024 x "
                     f"thresholds T=0.9/0.95/0.99, pinned slots (plain layout), gathers of {batch} distinct ids; "
                     f"value at W=1024, T=0.95; plus dense_gnn rows as fp16 (16384 x 128 half, HBM)",
         "rows": n, "tensor_bytes": L, "batch_ids": batch},
        savings_at, "ibp::k_decode_small", durs_at, link_roofline(link_at, durs_at, savings_at, None),
        sweep=points, fp16_dense_gnn=fp16)


WORKLOADS = {"sparse_gnn": run_sparse_gnn, "kv_bf16": run_kv_bf16, "dense_gnn": run_dense_gnn,
             "dlrm": run_dlrm, "llm_bf16": run_llm_bf16, "sparse_gnn_cache": run_sparse_gnn_cache,
             "sweep": run_sweep}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="sparse_gnn", choices=sorted(WORKLOADS))
    ap.add_argument("--small", action="store_true", help="scaled-down table (quick check)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-raw", action="store_true", help="skip the raw zero-copy gather comparison")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle decode")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the codec path is single-GPU; how it would shard across GPUs is a design note only)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    defaults = {"sparse_gnn": (200, 10), "kv_bf16": (100, 5), "dense_gnn": (200, 10), "dlrm": (4, 1),
                "sparse_gnn_cache": (200, 10), "sweep": (30, 5),
                "llm_bf16": (3, 1)}
    d_steps, d_warm = defaults[args.workload]
    args.steps = d_steps if args.steps is None else args.steps
    args.warmup = d_warm if args.warmup is None else args.warmup
    ibp.lib()
    res = WORKLOADS[args.workload](args)
    # every workload exits before printing when a decoded output of its last
    # timed step differs from the source or the library latched an error
    res["output_verified"] = "decoded output of the last timed step equal to the source, byte for byte; no device error"
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
