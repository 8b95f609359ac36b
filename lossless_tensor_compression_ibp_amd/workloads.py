"""Seeded synthetic inputs for the five workloads the codec is measured on.

This module holds no codec arithmetic: it only draws numbers (numpy
``default_rng``) and lays them out as the tensors the method compresses.  The
oracle tests, the GPU parity tests and the benchmark all take their inputs
from here, so both sides of every comparison see the same bytes.

The workloads stand in for the unnamed "real datasets" of the summaries
(FR/KO summary, section "Contributions clés" / "주요 기여", item 4): dense and
sparse GNN node features, DLRM embedding rows, BF16 LLM weights and a BF16 KV
cache (section "Résultats").  Shapes, distributions, chunk widths and
thresholds are fixed per workload below; where the description leaves a
choice open the plainest reading is taken (std for N(mu, sigma), one chunk =
one 32-bit word unless stated, sample = the first 1,024 tensors, T = 0.95
unless stated).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DATA_SEED = 0
ID_SEED = 1


@dataclass(frozen=True)
class Workload:
    name: str
    tensor_bytes: int  # L
    chunk_bits: int  # W
    period_bits: int  # M
    threshold: float  # T
    n_tensors: int
    n_sample: int  # tensors [0, n_sample) are the metadata sample
    location: str  # where the slots live when decoded: "hbm" or "host"


# Dense GNN node features: one 128 x fp32 row per tensor, one word per chunk.
DENSE_GNN = Workload("dense_gnn", 512, 32, 4096, 0.95, 16384, 1024, "hbm")
# Sparse GNN features: 256 x fp32 rows, chunk = 32 consecutive words.
SPARSE_GNN = Workload("sparse_gnn", 1024, 1024, 8192, 0.95, 1048576, 1024, "host")
# DLRM embedding table: 128 x fp32 rows, T = 0.9.
DLRM = Workload("dlrm", 512, 32, 4096, 0.90, 4194304, 1024, "host")
# LLM BF16 weights: one 4096 x 11008 layer per tensor, one Mask word shared
# by every chunk (a per-position Mask would be as large as a layer).
LLM_BF16 = Workload("llm_bf16", 4096 * 11008 * 2, 32, 32, 0.95, 32, 1, "host")
# BF16 KV cache: a page (16 tokens x 128 dims of one layer/head) per tensor.
KV_BF16 = Workload("kv_bf16", 4096, 32, 32768, 0.95, 262144, 1024, "hbm")

ALL = {w.name: w for w in (DENSE_GNN, SPARSE_GNN, DLRM, LLM_BF16, KV_BF16)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs).
    Works in place on a float32 array it may overwrite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = np.right_shift(u, np.uint32(16))
    np.bitwise_and(lsb, np.uint32(1), out=lsb)
    np.add(u, lsb, out=u)
    np.add(u, np.uint32(0x7FFF), out=u)
    np.right_shift(u, np.uint32(16), out=u)
    return u.astype(np.uint16)


def dense_gnn(n_rows: int = DENSE_GNN.n_tensors, seed: int = DATA_SEED) -> np.ndarray:
    """|N(0, 0.5)| fp32 rows of 128; round(3 %) of the rows replaced by N(0, 50)."""
    rng = np.random.default_rng(seed)
    x = np.abs(rng.normal(0.0, 0.5, size=(n_rows, 128))).astype(np.float32)
    n_out = int(round(0.03 * n_rows))
    rows = rng.choice(n_rows, size=n_out, replace=False)
    x[rows] = rng.normal(0.0, 50.0, size=(n_out, 128)).astype(np.float32)
    return x


def sparse_gnn(n_rows: int = SPARSE_GNN.n_tensors, seed: int = DATA_SEED,
               out: np.ndarray | None = None) -> np.ndarray:
    """256 fp32 per row; each entry non-zero with probability 0.03, non-zeros
    uniform in (0, 1].  Drawn in blocks of rows so ``out`` may be a pinned
    buffer of the full size."""
    rng = np.random.default_rng(seed)
    if out is None:
        out = np.empty((n_rows, 256), np.float32)
    block = 65536
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        nz = rng.random((r1 - r0, 256), dtype=np.float32) < np.float32(0.03)
        vals = np.float32(1.0) - rng.random(int(nz.sum()), dtype=np.float32)
        blk = np.zeros((r1 - r0, 256), np.float32)
        blk[nz] = vals
        out[r0:r1] = blk
    return out


def dlrm(n_rows: int = DLRM.n_tensors, seed: int = DATA_SEED,
         out: np.ndarray | None = None) -> np.ndarray:
    """128 fp32 per row, U(-0.01, 0.01) like an embedding initialisation."""
    rng = np.random.default_rng(seed)
    if out is None:
        out = np.empty((n_rows, 128), np.float32)
    block = 262144
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        u = rng.random((r1 - r0, 128), dtype=np.float32)
        out[r0:r1] = u * np.float32(0.02) - np.float32(0.01)
    return out


def llm_layer(layer: int, rows: int = 4096, cols: int = 11008, seed: int = DATA_SEED) -> np.ndarray:
    """One weight layer as bf16 bit patterns (uint16, rows x cols): N(0, 0.02),
    round(0.1 %) of the columns (channels) scaled by 20 before rounding."""
    rng = np.random.default_rng([seed, layer])
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(0.02)
    n_ch = max(1, int(round(0.001 * cols)))
    ch = rng.choice(cols, size=n_ch, replace=False)
    w[:, ch] *= np.float32(20.0)
    return to_bf16_bits(w)


def llm_layers(out: np.ndarray, rows: int = 4096, cols: int = 11008, seed: int = DATA_SEED,
               threads: int = 8) -> np.ndarray:
    """All layers into out (layers x rows*cols*2 bytes); layers are drawn from
    independent seeds, so drawing them on several threads gives the same bytes."""
    from concurrent.futures import ThreadPoolExecutor

    def one(l):
        out[l] = llm_layer(l, rows, cols, seed).reshape(-1).view(np.uint8)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(out.shape[0])))
    return out


def kv_cache(n_layers: int = 32, n_heads: int = 32, n_tokens: int = 4096, head_dim: int = 128,
             seed: int = DATA_SEED, out: np.ndarray | None = None) -> np.ndarray:
    """KV cache as bf16 bit patterns, shape (layers, heads, tokens, dim):
    N(0, 1) times a per-(layer, head, dim) scale drawn from lognormal(0, 1).
    Pages of 16 tokens x dim of one (layer, head) are contiguous 4 KiB blocks
    (page order: layer, head, token block)."""
    rng = np.random.default_rng(seed)
    if out is None:
        out = np.empty((n_layers, n_heads, n_tokens, head_dim), np.uint16)
    scale = rng.lognormal(0.0, 1.0, size=(n_layers, n_heads, head_dim)).astype(np.float32)
    for l in range(n_layers):
        z = rng.standard_normal((n_heads, n_tokens, head_dim), dtype=np.float32)
        z *= scale[l][:, None, :]
        out[l] = to_bf16_bits(z)
    return out


def batch_ids(n_rows: int, batch: int, n_batches: int, replace: bool, seed: int = ID_SEED):
    """Row-id batches (int64): distinct ids per batch when replace is False."""
    rng = np.random.default_rng(seed)
    out = np.empty((n_batches, batch), np.int64)
    for b in range(n_batches):
        if replace:
            out[b] = rng.integers(0, n_rows, size=batch, dtype=np.int64)
        else:
            out[b] = rng.choice(n_rows, size=batch, replace=False)
    return out
