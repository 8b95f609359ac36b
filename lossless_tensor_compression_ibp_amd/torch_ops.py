"""PyTorch operator registration over the C ABI (FR/KO summary, "Contributions
clés": the method ships as PyTorch extensions over GPU libraries, and a
framework integration takes a few lines of Python).

The ops live in the ``ibp`` namespace (``torch.ops.ibp.*``) and forward to the
binding in ``ibp.py``; every byte of codec work runs in libibp.so.  A handle
(``ibp.Meta``) cannot cross the operator boundary, so ``register(meta)``
returns an integer key that the ops take instead.  Each op also has a fake
(shape-only) implementation, so graphs that call it can be traced.

    from lossless_tensor_compression_ibp_amd import ibp, torch_ops
    key = torch_ops.register(ibp.ibp_build_metadata(sample, 1024, L, W, M, T))
    slots, bitmask, stored = torch.ops.ibp.compress(key, rows)
    batch = torch.ops.ibp.gather_decompress(key, slots, bitmask, ids)
"""
from __future__ import annotations

import itertools
import threading

import torch

from . import ibp

_lock = threading.Lock()
_handles: dict[int, ibp.Meta] = {}
_next = itertools.count(1)


def register(meta: ibp.Meta) -> int:
    """Key under which the ops find `meta` (kept alive until release())."""
    with _lock:
        key = next(_next)
        _handles[key] = meta
    return key


def release(key: int) -> None:
    with _lock:
        _handles.pop(key, None)


def _meta(key: int) -> ibp.Meta:
    try:
        return _handles[key]
    except KeyError:
        raise ValueError(f"no IBP handle registered under key {key}") from None


def _tensor_bytes(key: int) -> int:
    params, _, _ = ibp.ibp_meta_get(_meta(key))
    return int(params["tensor_bytes"])


def _check_status(meta: ibp.Meta) -> None:
    st = ibp.ibp_check(meta)
    if st != ibp.IBP_OK:
        raise ibp.IBPError(st, "device-side check")


@torch.library.custom_op("ibp::compress", mutates_args=())
def compress(key: int, src: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """src: uint8 (n, L) on the GPU or pinned.  Returns (slots (n, L) uint8 on
    src's side, bitmask int32 (ceil(n/32),) and stored bytes int64 (n,) on the
    GPU)."""
    meta = _meta(key)
    n = src.shape[0]
    dev = torch.device("cuda", torch.cuda.current_device())
    if src.is_cuda:
        slots = torch.empty_like(src)
    else:
        slots = torch.empty(src.shape, dtype=torch.uint8, pin_memory=True)
    bitmask = torch.zeros(max(1, (n + 31) // 32), dtype=torch.int32, device=dev)
    stored = torch.zeros(n, dtype=torch.int64, device=dev)
    ibp.ibp_compress(meta, src, n, slots, bitmask, stored)
    return slots, bitmask, stored


@compress.register_fake
def _(key: int, src: torch.Tensor):
    n = src.shape[0]
    dev = src.device if src.is_cuda else torch.device("cuda")
    return (torch.empty_like(src), torch.empty(max(1, (n + 31) // 32), dtype=torch.int32, device=dev),
            torch.empty(n, dtype=torch.int64, device=dev))


@torch.library.custom_op("ibp::decompress", mutates_args=())
def decompress(key: int, slots: torch.Tensor, bitmask: torch.Tensor) -> torch.Tensor:
    """All n slots decoded into a new (n, L) uint8 tensor on the GPU."""
    meta = _meta(key)
    n = slots.shape[0]
    out = torch.empty((n, _tensor_bytes(key)), dtype=torch.uint8, device=bitmask.device)
    ibp.ibp_decompress(meta, slots, bitmask, n, out)
    return out


@decompress.register_fake
def _(key: int, slots: torch.Tensor, bitmask: torch.Tensor):
    return torch.empty((slots.shape[0], slots.shape[1]), dtype=torch.uint8, device=bitmask.device)


@torch.library.custom_op("ibp::gather_decompress", mutates_args=())
def gather_decompress(key: int, slots: torch.Tensor, bitmask: torch.Tensor, ids: torch.Tensor) -> torch.Tensor:
    """Rows ids (int64, GPU) of the slots decoded into a new (len(ids), L)
    uint8 tensor on the GPU."""
    meta = _meta(key)
    out = torch.empty((ids.numel(), _tensor_bytes(key)), dtype=torch.uint8, device=ids.device)
    ibp.ibp_gather_decompress(meta, slots, slots.shape[0], bitmask, ids, out)
    return out


@gather_decompress.register_fake
def _(key: int, slots: torch.Tensor, bitmask: torch.Tensor, ids: torch.Tensor):
    return torch.empty((ids.numel(), slots.shape[1]), dtype=torch.uint8, device=ids.device)


def check(key: int) -> None:
    """Raises if a kernel latched an error (an id out of range, a corrupt
    record) since the last check; waits for the current stream."""
    _check_status(_meta(key))
