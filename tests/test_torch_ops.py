"""torch.ops.ibp.* registration: schemas and fake (shape-only) kernels on the
CPU, and agreement with the direct binding on the GPU."""
from __future__ import annotations

import numpy as np
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

from lossless_tensor_compression_ibp_amd import torch_ops  # noqa: F401  (registers the ops)


def test_ops_are_registered_with_their_schemas():
    for name in ("compress", "decompress", "gather_decompress"):
        op = getattr(torch.ops.ibp, name)
        schema = str(op.default._schema)
        assert schema.startswith(f"ibp::{name}(SymInt key, Tensor "), schema


def test_fake_kernels_give_the_output_shapes():
    with FakeTensorMode(allow_non_fake_inputs=False) as mode:
        slots = torch.empty((100, 512), dtype=torch.uint8, device="cuda")
        bm = torch.empty(4, dtype=torch.int32, device="cuda")
        ids = torch.empty(37, dtype=torch.int64, device="cuda")
        g = torch.ops.ibp.gather_decompress(1, slots, bm, ids)
        d = torch.ops.ibp.decompress(1, slots, bm)
        s, b, st = torch.ops.ibp.compress(1, slots)
    assert tuple(g.shape) == (37, 512) and g.dtype == torch.uint8
    assert tuple(d.shape) == (100, 512)
    assert tuple(s.shape) == (100, 512) and tuple(b.shape) == (4,) and tuple(st.shape) == (100,)
    del mode


def test_unknown_key_is_an_error():
    with pytest.raises(ValueError):
        torch_ops._meta(10**9)


@pytest.mark.gpu
def test_ops_match_the_binding_on_the_gpu():
    from lossless_tensor_compression_ibp_amd import ibp
    from lossless_tensor_compression_ibp_amd import workloads as WL

    w = WL.DENSE_GNN
    raw = np.ascontiguousarray(WL.dense_gnn(3000)).view(np.uint8).reshape(3000, -1)
    src = torch.from_numpy(raw).cuda()
    meta = ibp.ibp_build_metadata(src, 1024, raw.shape[1], w.chunk_bits, w.period_bits, w.threshold)
    key = torch_ops.register(meta)
    slots, bm, stored = torch.ops.ibp.compress(key, src)
    ref_slots = torch.empty_like(src)
    ref_bm = torch.zeros_like(bm)
    ref_st = torch.zeros_like(stored)
    ibp.ibp_compress(meta, src, src.shape[0], ref_slots, ref_bm, ref_st)
    assert torch.equal(bm, ref_bm) and torch.equal(stored, ref_st)
    for t in range(0, 3000, 97):
        k = int(ref_st[t])
        assert torch.equal(slots[t, :k], ref_slots[t, :k])
    assert torch.equal(torch.ops.ibp.decompress(key, slots, bm), src)
    ids = torch.from_numpy(np.random.default_rng(2).integers(0, 3000, 999)).cuda()
    assert torch.equal(torch.ops.ibp.gather_decompress(key, slots, bm, ids), src[ids])
    torch_ops.check(key)
    torch.library.opcheck(torch.ops.ibp.gather_decompress.default, (key, slots, bm, ids),
                          test_utils=("test_schema", "test_faketensor"))
    torch_ops.release(key)
