"""IBP decode benchmark on one MI355X.

Default (--workload all): every workload at its full size, one after the
other, and ONE JSON line on stdout.  Its headline is the largest workload,
llm_bf16 (32 layers of 4096 x 11008 bf16 weights, 2.89 GB per pass, held
compressed in pinned host memory and decoded zero-copy into HBM one layer at
a time while a consumer reads the previous layer); the other workloads
(sparse_gnn, dlrm, kv_bf16, dense_gnn, sparse_gnn_cache) are nested under
"workloads", each with its own decoded GB/s, space savings, roofline of its
decode kernel and CPU oracle baseline.

Per workload: decoded GB/s of uncompressed output (the metric), space
savings, the decode kernel's algorithmic bytes per launch over its average
launch duration (HIP events on its stream) against the roofline that bounds
it (host link: PCIe 5.0 x16, 64 GB/s per direction, with the hipMemcpy H2D
ceiling measured in the same run; HBM: 8 TB/s), the encode rate against the
same bound, and the CPU oracle timed on a bounded sample, single-threaded and
on every core the process may use.

--workload NAME runs one workload alone (sparse_gnn, dlrm, kv_bf16,
dense_gnn, sparse_gnn_cache, llm_bf16, or the W x T sweep).
"""
from __future__ import annotations

import argparse
import copy
import gc
import json
import os
import sys
import threading
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
LINE = 128              # bytes a zero-copy read of pinned host memory moves at a time
METRIC = "IBP decode GB/s (uncompressed out, 1 MI355X) + % of roofline + space savings %"


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with runs of white space
    collapsed (string literals are kept as they are)."""
    import re

    token = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)
    text = token.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored); counter
    readings in profiles/traffic.json apply only while it matches."""
    import glob
    import hashlib

    csrc = os.path.join(ROOT, "lossless_tensor_compression_ibp_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp")))
    files.append(os.path.join(ROOT, "include", "ibp.h"))
    h = hashlib.sha256()
    for f in sorted(files, key=os.path.basename):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


TRAFFIC_SOURCE = ("copied from profiles/traffic.json: rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE of a separate "
                  "run of this workload (KiB per dispatch, one counter per run), each scaled by what the counter "
                  "reads for a copy of known size with the same access pattern; null when the kernel sources changed "
                  "since the counters were taken")
TRAFFIC_SUMS_LINK = ("bytes per launch: reads over the host link (whole 128-byte lines) + HBM reads of ids, bitmask and "
                     "header words + HBM writes of the decoded rows")
TRAFFIC_SUMS_HBM = "bytes per launch: HBM reads + HBM writes"


def measured_traffic(workload: str | None):
    """(traffic bytes per launch, read bytes per launch) of the workload's
    decode kernel from the committed rocprofv3 counter runs, or (None, None)
    when the kernels changed since the counters were taken."""
    if workload is None:
        return None, None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("source_hash") != kernel_source_hash():
        return None, None
    entry = t.get("workloads", {}).get(workload)
    if entry is None:
        return None, None
    return entry.get("traffic_bytes_per_launch"), entry.get("read_bytes_per_launch")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def pinned(shape, dtype):
    return torch.empty(shape, dtype=dtype, pin_memory=True)


def line_bytes(stored: np.ndarray) -> int:
    """Bytes a zero-copy read of these stored items moves: whole 128-byte
    lines (every slot starts on a line boundary)."""
    return int((LINE * ((np.asarray(stored, dtype=np.int64) + LINE - 1) // LINE)).sum())


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


RAMP_S = 0.25  # untimed calls before the warm-up, so the GPU's clocks have ramped up (--ramp)


def ramp(fn):
    """Calls fn(0) until RAMP_S seconds of wall time have passed
    (synchronising every call): short timed regions (a few ms) otherwise
    start on a GPU whose clocks are still rising from idle."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < RAMP_S:
        fn(0)
        torch.cuda.synchronize()


def timed(fn, steps: int, warmup: int):
    """Runs fn(i) warmup times (after the untimed ramp), then times exactly
    `steps` calls between two synchronisations.  Returns (wall seconds,
    launch durations in seconds): one HIP event pair on the launching stream
    brackets the whole timed region, and each launch is credited the region's
    GPU time / steps (events around every launch would put their own gaps
    between the kernels)."""
    stream = torch.cuda.current_stream()
    ramp(fn)
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


# ---------------------------------------------------------------------------
# CPU oracle baselines: the oracle as it stands, single-threaded, and the same
# oracle on every core the process may use over disjoint tensor ranges
# ---------------------------------------------------------------------------
def oracle_threads() -> int:
    """Threads for the all-cores baseline: the cores this process may run on,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run_threads(work, n_threads: int, budget_s: float):
    """work(k, deadline) -> bytes thread k decoded; the oracle's C calls
    release the GIL, so the threads run on separate cores.  Returns (total
    bytes, wall seconds)."""
    out = [0] * n_threads
    t0 = time.perf_counter()
    deadline = t0 + budget_s

    def one(k):
        out[k] = work(k, deadline)

    ts = [threading.Thread(target=one, args=(k,)) for k in range(n_threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(out), time.perf_counter() - t0


def cpu_gather_baseline(rows: np.ndarray, w: WL.Workload, batch: int, budget_s: float, what: str,
                        layout: str = "slots", replace: bool = True) -> dict:
    """Gathers of random id batches decoded by the oracle from its own slots
    ("slots"), slots with headers in a separate array ("split") or packed
    items ("packed") of `rows` (encode excluded): single-threaded for
    budget_s, then on every core over disjoint row ranges for budget_s / 2."""
    from oracle import oracle

    oracle.build(force=False)
    rows = np.ascontiguousarray(rows)
    n, L = rows.shape
    W, M = w.chunk_bits, w.period_bits
    ns = min(w.n_sample, n)
    mask, bitval = oracle.build_metadata(rows[:ns], 8 * L, W, M, w.threshold, ns)
    if layout == "split":
        slots, headers, bm, _ = oracle.compress_split(rows, L, W, M, mask, bitval, n)
        gather = lambda ids: oracle.gather_decompress_split(slots, n, headers, bm, ids, L, W, M, mask, bitval)  # noqa: E731
    elif layout == "packed":
        buf, off, bm = oracle.compress_packed(rows, L, W, M, mask, bitval, n)
        gather = lambda ids: oracle.gather_decompress_packed(buf, off, n, bm, ids, L, W, M, mask, bitval)  # noqa: E731
    else:
        slots, bm, _ = oracle.compress(rows, L, W, M, mask, bitval, n)
        gather = lambda ids: oracle.gather_decompress(slots, n, bm, ids, L, W, M, mask, bitval)  # noqa: E731

    def draw(rng, lo, hi, b):
        return lo + (rng.choice(hi - lo, b, replace=False) if not replace else rng.integers(0, hi - lo, b))

    rng = np.random.default_rng(WL.ID_SEED)
    done = 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        ids = draw(rng, 0, n, batch)
        out = gather(ids)
        done += batch
    dt = time.perf_counter() - t0
    if not np.array_equal(out, rows[ids]):
        raise SystemExit("oracle gather differs from the source rows")
    P = oracle_threads()

    def work(k, deadline):
        lo, hi = k * n // P, (k + 1) * n // P
        b = min(batch, hi - lo)
        r = np.random.default_rng([WL.ID_SEED, k])
        got = 0
        while got == 0 or time.perf_counter() < deadline:
            gather(draw(r, lo, hi, b))
            got += b * L
        return got

    tot, wall = run_threads(work, P, budget_s / 2)
    return {"value": round(done * L / dt / GB, 6), "unit": "GB/s", "cores": 1, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{done} rows decoded by gather in batches of {batch} ids from the oracle's "
                      f"{ {'split': 'slots (headers in a separate array)', 'packed': 'packed items'}.get(layout, 'slots')} "
                      f"of {what} ({dt:.1f} s, single thread)",
            "all_cores": {"value": round(tot / wall / GB, 6), "unit": "GB/s", "cores": P, "kind": "oracle",
                          "sample": f"the same gathers on {P} threads, thread k drawing ids from its own 1/{P} of the "
                                    f"rows ({wall:.1f} s); a baseline only"}}


def cpu_roundtrip_baseline(rows: np.ndarray, w: WL.Workload, n_sample: int, budget_s: float, what: str,
                           single_n: int | None = None) -> dict:
    """The oracle single-threaded: metadata from the first n_sample rows, then
    compress and decompress of the first single_n rows (default all) until
    budget_s is spent (value: decode GB/s, encode_GBps beside it); then decode
    of its own slots of all the rows on every core, thread k on its own 1/P of
    them, for budget_s / 2."""
    from oracle import oracle

    oracle.build(force=False)
    rows = np.ascontiguousarray(rows)
    n, L = rows.shape
    W, M = w.chunk_bits, w.period_bits
    mask, bitval = oracle.build_metadata(rows[:n_sample], 8 * L, W, M, w.threshold, n_sample)
    n1 = n if single_n is None else single_n
    t_enc = t_dec = 0.0
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        a = time.perf_counter()
        slots, bm, _ = oracle.compress(rows[:n1], L, W, M, mask, bitval, n1)
        b = time.perf_counter()
        out = oracle.decompress(slots, bm, L, W, M, mask, bitval, n1)
        t_enc += b - a
        t_dec += time.perf_counter() - b
        reps += 1
    if not np.array_equal(out, rows[:n1]):
        raise SystemExit("oracle round trip differs")
    P = oracle_threads()
    per = max(1, n // P)
    parts = [(k * per, min(n, (k + 1) * per)) for k in range(min(P, n))]
    enc = [None] * len(parts)

    def encode_part(k, deadline):  # untimed set-up, on all threads too
        lo, hi = parts[k]
        enc[k] = oracle.compress(rows[lo:hi], L, W, M, mask, bitval, hi - lo)[:2]
        return 0

    run_threads(encode_part, len(parts), 0.0)

    def work(k, deadline):
        lo, hi = parts[k]
        sl, bmk = enc[k]
        got = 0
        while got == 0 or time.perf_counter() < deadline:
            oracle.decompress(sl, bmk, L, W, M, mask, bitval, hi - lo)
            got += (hi - lo) * L
        return got

    tot, wall = run_threads(work, len(parts), budget_s / 2)
    return {"value": round(reps * n1 * L / t_dec / GB, 6), "unit": "GB/s", "cores": 1, "host_cores": os.cpu_count(),
            "kind": "oracle", "encode_GBps": round(reps * n1 * L / t_enc / GB, 6),
            "sample": f"{what}: {reps} compress + decompress round trips ({t_enc + t_dec:.1f} s, single thread)",
            "all_cores": {"value": round(tot / wall / GB, 6), "unit": "GB/s", "cores": len(parts), "kind": "oracle",
                          "sample": f"decode of the oracle's own slots of all {n} tensors of the sample on "
                                    f"{len(parts)} threads, thread k on its own 1/{len(parts)} of them ({wall:.1f} s); "
                                    f"a baseline only"}}


# ---------------------------------------------------------------------------
# Result assembly
# ---------------------------------------------------------------------------
def base_result(args, value, wall, config, savings, kernel, durs, roofline, **extra) -> dict:
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": config, "space_savings_pct": round(100 * savings, 3), "kernel": kernel,
        "kernel_avg_us": round(float(np.mean(durs)) * 1e6, 2), "roofline": roofline,
        "ramp_s": RAMP_S,
    }
    res.update(extra)
    return res


def hbm_roofline(bytes_per_launch: float, durs, workload: str | None) -> dict:
    achieved = bytes_per_launch / float(np.mean(durs)) / GB
    traffic, _ = measured_traffic(workload)
    return {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_source": TRAFFIC_SOURCE,
            "traffic_sums": TRAFFIC_SUMS_HBM, "copy_kernel_ceiling_measured": round(copy_kernel_ceiling(), 3),
            "algorithmic_bytes_per_launch": int(bytes_per_launch)}


def link_roofline(link_bytes_per_launch: float, durs, savings: float, workload: str | None, h2d: float,
                  line_bytes_per_launch: float | None = None, out_bytes_per_launch: float | None = None) -> dict:
    """Host-link roofline of a zero-copy decode: record bytes over the link
    per launch / launch duration against 64 GB/s, with the same-run H2D
    ceiling; the decoded roofline is H2D / compressed fraction, and, where
    whole 128-byte lines are what the link moves, H2D x output / line bytes."""
    achieved = link_bytes_per_launch / float(np.mean(durs)) / GB
    traffic, read = measured_traffic(workload)
    r = {"bound": "pcie", "achieved": round(achieved, 3), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
         "frac": round(achieved / PCIE5_X16_GBPS, 4), "traffic": traffic, "traffic_source": TRAFFIC_SOURCE,
         "traffic_sums": TRAFFIC_SUMS_LINK, "traffic_read_bytes": read,
         "link_ceiling_measured": round(h2d, 3), "frac_of_measured_ceiling": round(achieved / h2d, 4),
         "algorithmic_bytes_per_launch": int(link_bytes_per_launch),
         "decoded_roofline_GBps": round(h2d / (1.0 - savings), 3)}
    if line_bytes_per_launch is not None and out_bytes_per_launch:
        r["line_bytes_per_launch"] = int(line_bytes_per_launch)
        r["line_granular_decoded_roofline_GBps"] = round(h2d * out_bytes_per_launch / line_bytes_per_launch, 3)
    return r


def decoded_fracs(res: dict):
    """Decoded GB/s against the decoded rooflines of a link-bound line."""
    roof = res["roofline"]
    res["decoded_frac_of_roofline"] = round(res["value"] / roof["decoded_roofline_GBps"], 4)
    res["decoded_frac_of_published_link_roofline"] = round(
        res["value"] / (PCIE5_X16_GBPS / (1.0 - res["space_savings_pct"] / 100)), 4)
    if "line_granular_decoded_roofline_GBps" in roof:
        res["decoded_frac_of_line_granular_roofline"] = round(
            res["value"] / roof["line_granular_decoded_roofline_GBps"], 4)


def encode_link(in_bytes: float, seconds: float, h2d: float, note: str) -> dict:
    gbps = in_bytes / seconds / GB
    return {"GBps": round(gbps, 3), "bound": "pcie", "frac_of_measured_h2d": round(gbps / h2d, 4),
            "frac_of_peak": round(gbps / PCIE5_X16_GBPS, 4), "note": note}


def encode_hbm(in_bytes: float, hbm_bytes: float, seconds: float, note: str) -> dict:
    return {"GBps": round(in_bytes / seconds / GB, 3), "bound": "hbm",
            "hbm_GBps": round(hbm_bytes / seconds / GB, 3),
            "frac_of_peak": round(hbm_bytes / seconds / GB / HBM_PEAK_GBPS, 4), "note": note}


# ---------------------------------------------------------------------------
# Sparse GNN: zero-copy gather from pinned host slots
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
    t_enc = encode_seconds(lambda: ibp.ibp_compress_split(meta, host, n, slots, headers, bitmask, stored))
    payload_np = stored.cpu().numpy()
    comp_np = (bitmask.cpu().numpy().view(np.uint32)[np.arange(n) >> 5] >> (np.arange(n) & 31)) & 1
    # compressed bytes: payload in the slots plus the header words kept in HBM
    savings = 1.0 - (payload_np.sum() + 4 * hw * comp_np.sum()) / (n * L)

    log("[bench] the plain slot layout (header in the slot) for comparison")
    slots_plain = pinned((n, L), torch.uint8)
    bitmask_plain = torch.zeros_like(bitmask)
    stored_plain = torch.zeros(n, dtype=torch.int64, device=dev)
    t_enc_plain = encode_seconds(lambda: ibp.ibp_compress(meta, host, n, slots_plain, bitmask_plain, stored_plain))
    stored_plain_np = stored_plain.cpu().numpy()
    savings_plain = 1.0 - stored_plain_np.sum() / (n * L)

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

    raw_wall = float("nan") if args.no_raw else timed(raw_step, args.steps, args.warmup)[0]
    h2d = h2d_ceiling()
    roof = link_roofline(float(link_bytes.mean()), durs, savings, None if args.small else "sparse_gnn", h2d,
                         float(np.mean([line_bytes(payload_np[t]) for t in timed_ids])), out_bytes)
    plain_link = float(stored_plain_np[timed_ids].sum(axis=1).mean())
    plain_lines = float(np.mean([line_bytes(stored_plain_np[t]) for t in timed_ids]))
    plain_value = args.steps * out_bytes / plain_wall / GB
    plain_achieved = plain_link / float(plain_durs.mean()) / GB
    res = base_result(
        args, value, wall,
        {"workload": f"sparse_gnn: {n} rows x 256 fp32 (97% zeros), W=1024, M=8192, T=0.95, 1 KiB slots in pinned "
                     f"host memory (payload only; each compressed row's header word in HBM beside the bitmask), "
                     f"zero-copy gather of {batch} distinct random row ids per step into HBM",
         "rows": n, "tensor_bytes": L, "batch_ids": batch, "chunk_bits": w.chunk_bits,
         "period_bits": w.period_bits, "threshold": w.threshold, "layout": "headers in HBM",
         "hbm_header_bytes": int(4 * hw * n), "hbm_bitmask_bytes": int(4 * ((n + 31) // 32)),
         "hbm_header_bytes_read_per_launch": int(4 * hw * batch)},
        savings, "ibp::k_decode_small<0, true, true, 1, true>", durs, roof,
        slot_layout={
            "what": "the pages' own layout: the whole record (header word + payload) in the slot, only the bitmask "
                    "in HBM; same rows, same ids, same run",
            "decoded_GBps": round(plain_value, 3), "kernel_avg_us": round(float(plain_durs.mean()) * 1e6, 2),
            "space_savings_pct": round(100 * savings_plain, 3),
            "link_bytes_per_launch": int(plain_link), "line_bytes_per_launch": int(plain_lines),
            "achieved_GBps": round(plain_achieved, 3), "frac_of_peak": round(plain_achieved / PCIE5_X16_GBPS, 4),
            "frac_of_measured_ceiling": round(plain_achieved / h2d, 4),
            "decoded_frac_of_roofline": round(plain_value / (h2d / (1.0 - savings_plain)), 4),
            "decoded_frac_of_line_granular_roofline": round(plain_value / (h2d * out_bytes / plain_lines), 4),
            "encode": encode_link(n * L, t_enc_plain, h2d, "host -> host, pinned source to pinned slots")},
        raw_zero_copy_gather_GBps=round(args.steps * out_bytes / raw_wall / GB, 3),
        speedup_vs_raw_zero_copy=round(raw_wall / wall, 3),
        encode=encode_link(n * L, t_enc, h2d, "host -> host, pinned source to pinned slots, header words to HBM"),
        metadata_ms=round(t_meta * 1e3, 2), meta=info)
    decoded_fracs(res)
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_gather_baseline(raw_np[:16384], w, 1024, args.cpu_budget,
                                                  "the first 16,384 rows (16 MiB)", layout="split", replace=False)
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
    # compressed pages, and the chunks that matched in them (header bits)
    bits = np.unpackbits(bitmask.cpu().numpy().view(np.uint8), bitorder="little")[:n].astype(bool)
    hdr = slots[torch.from_numpy(np.flatnonzero(bits)).to(dev), :128].cpu().numpy().view(np.uint32)
    matched = int(np.bitwise_count(hdr).sum())
    out = torch.empty_like(src)
    wall, durs = timed(lambda i: ibp.ibp_decompress(meta, slots, bitmask, n, out), args.steps, args.warmup)
    assert ibp.ibp_check(meta) == ibp.IBP_OK
    if not torch.equal(out, src):
        raise SystemExit("decoded pages differ")
    hbm_bytes = float(stored_np.sum() + n * L + 4 * ((n + 31) // 32))
    roof = hbm_roofline(hbm_bytes, durs, None if args.small else "kv_bf16")
    t_enc = float(np.mean(enc_durs))
    res = base_result(
        args, n * L * args.steps / wall / GB, wall,
        {"workload": f"kv_bf16: {layers} layers x 32 heads x 4096 tokens x 128 bf16, 4 KiB pages in HBM slots, "
                     f"W=32, M=32768, T=0.95, decode of all {n} pages per step", "pages": n, "tensor_bytes": L},
        savings, "ibp::k_decode_small<3, false, true, 4, false>", durs, roof,
        compressed_page_frac=round(float(bits.mean()), 6),
        matched_chunk_frac_in_compressed_pages=round(matched / max(1, int(bits.sum()) * 1024), 6),
        encode=encode_hbm(n * L, n * L + stored_np.sum(), t_enc, "HBM -> HBM, all pages per launch"),
        metadata_ms=round(t_meta * 1e3, 2), meta=ibp.ibp_meta_get_info(meta))
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_roundtrip_baseline(
            src[:2048].cpu().numpy(), w, w.n_sample, args.cpu_budget,
            "the first 2,048 pages (8 MiB; metadata from their first 1,024)")
    return res


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
    timed(lambda i: ibp.ibp_compress(meta, src, n, slots, bitmask, stored), 20, 2)
    enc_durs = queued_durations(lambda i: ibp.ibp_compress(meta, src, n, slots, bitmask, stored), 20)
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
    res = base_result(
        args, n * L * args.steps / wall / GB, wall,
        {"workload": f"dense_gnn: {n} rows x 128 fp32 |N(0,0.5)| with 3% N(0,50) rows, W=32, M=4096, T=0.95, "
                     f"slots in HBM, contiguous decode of all rows per step", "rows": n, "tensor_bytes": L},
        savings, "ibp::k_decode_rows<1, false, 2, false, 2> (two rows per wave)", durs,
        hbm_roofline(hbm_bytes, durs, "dense_gnn"),
        encode=encode_hbm(n * L, n * L + stored_np.sum(), float(np.mean(enc_durs)), "HBM -> HBM, all rows per launch"),
        uncompressed_hbm_copy_GBps=round(n * L * args.steps / raw_wall / GB, 3),
        uncompressed_copy_kernel_us=round(float(np.mean(raw_durs)) * 1e6, 2), meta=ibp.ibp_meta_get_info(meta))
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_roundtrip_baseline(raw_np, w, w.n_sample, args.cpu_budget,
                                                     f"all {n} rows (8 MiB; metadata from the first 1,024)")
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
    timed_ids = ids_np[args.warmup * per_step:]
    link = float(stored_np[timed_ids].sum(axis=1).mean())
    lines = float(np.mean([line_bytes(stored_np[t]) for t in timed_ids[:per_step]]))
    value = args.steps * per_step * batch * L / wall / GB
    h2d = h2d_ceiling()
    res = base_result(
        args, value, wall,
        {"workload": f"dlrm: {n} rows x 128 fp32 U(-0.01,0.01), W=32, M=4096, T=0.9, slots in pinned host "
                     f"memory, {per_step} zero-copy gathers of {batch} random ids (with replacement) per step",
         "rows": n, "tensor_bytes": L, "batch_ids": batch, "gathers_per_step": per_step},
        savings, "ibp::k_decode_small<2, true, true, 0, false>", durs,
        link_roofline(link, durs, savings, None if args.small else "dlrm", h2d, lines, batch * L),
        line_granular_note=("a 512-byte row whose record is about 465 bytes still spans 4 lines of 128 bytes, "
                            "so at this saving the link moves the same lines as for raw rows"),
        encode=encode_link(n * L, t_enc, h2d, "host -> host, pinned source to pinned slots"),
        meta=ibp.ibp_meta_get_info(meta))
    decoded_fracs(res)
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_gather_baseline(raw_np[:65536], w, 8192, args.cpu_budget,
                                                  "the first 65,536 rows (32 MiB)")
    return res


# ---------------------------------------------------------------------------
# LLM BF16 weights: 32 layers streamed from pinned host slots, one layer of
# prefetch: decode of layer i+1 (stream A) overlaps a consumer of layer i
# (stream B, y = x @ W on the decoded layer)
# ---------------------------------------------------------------------------
LLM_KERNEL = "ibp::k_decode_groups<3, true, 8u, 2048u> (look-back over groups of 8 tiles of 8 KiB)"
LLM_HBM_KERNELS = ("ibp::k_group_bits<4u, 2048u> + ibp::k_group_scan + ibp::k_decode_groups<3, true, 4u, 2048u> "
                   "(group start bits from a pass over the header words, then groups of 4 tiles of 8 KiB; "
                   "kernel_avg_us spans all three)")


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
    marks = []
    prev_freed = []  # the consumer's events of the previous pass

    def one_pass(record: bool):
        ready = [torch.cuda.Event() for _ in range(layers)]
        freed = [torch.cuda.Event() for _ in range(layers)]
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(sa)
        for l in range(layers):
            with torch.cuda.stream(sa):
                # the buffer of layer l was last read by the consumer of layer l - 2
                if l >= 2:
                    sa.wait_event(freed[l - 2])
                elif prev_freed:
                    sa.wait_event(prev_freed[layers - 2 + l])
                ibp.ibp_gather_decompress(meta, slots, layers, bitmask, ids[l:l + 1], bufs[l & 1], stream=sa)
                ready[l].record(sa)
            with torch.cuda.stream(sb):
                sb.wait_event(ready[l])
                torch.matmul(x, bufs[l & 1].view(torch.bfloat16).view(rows, cols), out=y)
                freed[l].record(sb)
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(sa)
            marks.append((e0, e1))
        prev_freed[:] = freed

    ramp(lambda i: one_pass(False))
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
    # decode launch duration: the decode stream's span of a pass / layers (the
    # decode of layer l waits only for the consumer of layer l - 2, which
    # finishes long before; the launches run back to back)
    durs = np.array([a.elapsed_time(b) / 1e3 / layers for a, b in marks])
    link = float(stored_np.mean())
    value = args.steps * layers * L / wall / GB
    del bufs
    hbm_resident = None
    if not args.no_hbm_resident:
        # the same records already resident in HBM: one decode of all layers
        # per step, HBM -> HBM (no host link in the timed region)
        log("[bench] llm_bf16: the same layers decoded from HBM-resident slots")
        dslots = slots.to(dev)
        dout = torch.empty((layers, L), dtype=torch.uint8, device=dev)
        hbm_wall, hbm_durs = timed(lambda i: ibp.ibp_decompress(meta, dslots, bitmask, layers, dout), args.steps,
                                   args.warmup)
        assert ibp.ibp_check(meta) == ibp.IBP_OK
        if not np.array_equal(dout[layers - 1].cpu().numpy(), hv[layers - 1]):
            raise SystemExit("decoded layer (HBM-resident slots) differs")
        hbm_bytes = float(stored_np.sum() + layers * L + 4 * ((layers + 31) // 32))
        # the same layers encoded with source and slots in HBM; records equal
        # to those written to the pinned slots
        log("[bench] llm_bf16: the same layers encoded HBM -> HBM")
        dsrc = host.to(dev)
        eslots = torch.empty((layers, L), dtype=torch.uint8, device=dev)
        ebm, estored = torch.zeros_like(bitmask), torch.zeros_like(stored)
        t_enc_hbm = encode_seconds(lambda: ibp.ibp_compress(meta, dsrc, layers, eslots, ebm, estored))
        if not (torch.equal(ebm, bitmask) and torch.equal(estored, stored)) or not all(
                torch.equal(eslots[l, :int(stored_np[l])], dslots[l, :int(stored_np[l])]) for l in range(layers)):
            raise SystemExit("HBM -> HBM encode differs from the pinned-slot records")
        del dsrc, eslots
        hbm_resident = {
            "what": f"the same {layers} compressed layers held in HBM slots, all of them decoded by one "
                    f"ibp_decompress per step into HBM (inputs resident in HBM, no host link)",
            "decoded_GBps": round(args.steps * layers * L / hbm_wall / GB, 3),
            "ms_per_step": round(hbm_wall / args.steps * 1e3, 4), "kernel": LLM_HBM_KERNELS,
            "kernel_avg_us": round(float(np.mean(hbm_durs)) * 1e6, 2),
            "roofline": hbm_roofline(hbm_bytes, hbm_durs, "llm_bf16_hbm"),
            "encode": encode_hbm(layers * L, layers * L + float(stored_np.sum()), t_enc_hbm,
                                 "HBM -> HBM, source and slots in device memory: a first pass sums each group of "
                                 "4 tiles' payload bits, a scan gives the start bits, then one wave encodes a "
                                 "group")}
        del dslots, dout
    h2d = h2d_ceiling()
    res = base_result(
        args, value, wall,
        {"workload": f"llm_bf16: {layers} layers of {rows}x{cols} bf16 N(0,0.02) (0.1% columns x20), W=32, M=32, "
                     f"T=0.95, slots in pinned host memory, each layer decoded zero-copy into HBM on one stream "
                     f"while a consumer (y = x @ W) reads the previous layer on another", "layers": layers,
         "tensor_bytes": L},
        savings, LLM_KERNEL, durs,
        link_roofline(link, durs, savings, None if args.small else "llm_bf16", h2d),
        hbm_resident=hbm_resident,
        encode=encode_link(layers * L, t_enc, h2d, "host -> host, pinned source to pinned slots"),
        meta=ibp.ibp_meta_get_info(meta))
    decoded_fracs(res)
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        # layer 0 cut into 16 tensors of 256 rows (5.6 MB each), metadata from
        # the first; one of them single-threaded, all 16 on every core
        res["cpu_baseline"] = cpu_roundtrip_baseline(
            hv[0].reshape(16, -1), w, 1, args.cpu_budget,
            "one 5.6 MB tensor: the first 256 rows of layer 0 (metadata from itself)", single_n=1)
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
    h2d = h2d_ceiling()
    fill = float(np.median(fill_s))
    res = base_result(
        args, batch * L * args.steps / wall / GB, wall,
        {"workload": f"sparse_gnn_cache: {n} rows x 256 fp32 (97% zeros), W=1024, M=8192, T=0.95, all rows "
                     f"compressed into one packed HBM buffer (items back to back, 16-byte aligned), gather of "
                     f"{batch} distinct random row ids per step into HBM", "rows": n, "tensor_bytes": L,
         "batch_ids": batch},
        1.0 - total / (n * L), "ibp::k_decode_rows<0, true, 4, true, 2> (packed items, two rows per wave)", durs,
        hbm_roofline(hbm_bytes, durs, None if args.small else "sparse_gnn_cache"),
        cache_bytes=total, capacity_gain=round(n * L / total, 4),
        fill=dict(encode_link(2 * n * L, fill, h2d, "cache fill from pinned rows: the offsets pass, then the items "
                                                    "pass (two reads of the source over the link)"),
                  GBps=round(n * L / fill / GB, 3)),
        uncompressed_hbm_gather_GBps=round(batch * L * args.steps / raw_wall / GB, 3),
        uncompressed_gather_kernel_us=round(float(np.mean(raw_durs)) * 1e6, 2),
        meta=ibp.ibp_meta_get_info(meta))
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_gather_baseline(raw_np[:16384], w, 1024, args.cpu_budget,
                                                  "the first 16,384 rows (16 MiB)", layout="packed", replace=False)
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
        savings_at, "ibp::k_decode_small", durs_at, link_roofline(link_at, durs_at, savings_at, None, h2d_ceiling()),
        sweep=points, fp16_dense_gnn=fp16)


WORKLOADS = {"sparse_gnn": run_sparse_gnn, "kv_bf16": run_kv_bf16, "dense_gnn": run_dense_gnn,
             "dlrm": run_dlrm, "llm_bf16": run_llm_bf16, "sparse_gnn_cache": run_sparse_gnn_cache,
             "sweep": run_sweep}
# steps, warmup when the command line gives none
DEFAULT_STEPS = {"sparse_gnn": (200, 10), "kv_bf16": (100, 5), "dense_gnn": (200, 10), "dlrm": (4, 1),
                 "sparse_gnn_cache": (200, 10), "sweep": (30, 5), "llm_bf16": (3, 1)}
# the default run: the headline (largest workload) last
ALL_ORDER = ("dense_gnn", "sparse_gnn", "sparse_gnn_cache", "dlrm", "kv_bf16", "llm_bf16")
HEADLINE = "llm_bf16"
VERIFIED = "decoded output of the last timed step equal to the source, byte for byte; no device error"


def release_memory():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    host_empty = getattr(torch._C, "_host_emptyCache", None)
    if host_empty is not None:
        host_empty()


def run_one(name: str, args) -> dict:
    a = copy.copy(args)
    d_steps, d_warm = DEFAULT_STEPS[name]
    a.steps = d_steps if args.steps is None else args.steps
    a.warmup = d_warm if args.warmup is None else args.warmup
    log(f"[bench] === {name}: {a.steps} timed steps, {a.warmup} warm-up ===")
    t0 = time.perf_counter()
    res = WORKLOADS[name](a)
    # every workload exits before returning when a decoded output of its last
    # timed step differs from the source or the library latched an error
    res["output_verified"] = VERIFIED
    res["run_s"] = round(time.perf_counter() - t0, 1)
    release_memory()
    return res


def run_all(args) -> dict:
    results = {name: run_one(name, args) for name in ALL_ORDER}
    head = results.pop(HEADLINE)
    head["config"]["headline"] = ("the largest workload that fits one GPU: 32 bf16 layers, 2.89 GB of weights per "
                                  "pass; every other workload is nested under 'workloads'")
    common = ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data")
    head["workloads"] = {name: {k: v for k, v in r.items() if k not in common} for name, r in results.items()}
    return head


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS))
    ap.add_argument("--small", action="store_true", help="scaled-down tables (quick check)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-raw", action="store_true", help="skip the raw zero-copy gather comparison")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of single-thread oracle decode per workload (half that on all cores)")
    ap.add_argument("--no-hbm-resident", action="store_true",
                    help="llm_bf16: skip the decode of the same layers from HBM-resident slots")
    ap.add_argument("--ramp", type=float, default=RAMP_S,
                    help="seconds of untimed calls before each warm-up (clock ramp; 0 under a profiler)")
    args = ap.parse_args()
    globals()["RAMP_S"] = args.ramp
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the codec path is single-GPU; how it would shard across GPUs is a design note only)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ibp.lib()
    res = run_all(args) if args.workload == "all" else run_one(args.workload, args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
