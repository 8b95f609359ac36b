"""The C-ABI library loads on a machine without a GPU and exports every
function include/ibp.h declares (no compute calls here)."""
import ctypes
import os
import re

from lossless_tensor_compression_ibp_amd import ibp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "ibp.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ibp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_functions():
    assert declared_functions() == sorted(ibp.ABI_FUNCTIONS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ibp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_host_side_argument_checks():
    L = ibp.lib()
    assert ibp.status_string(0) == "ok"
    assert ibp.status_string(ibp.IBP_ERR_CORRUPT) == "corrupt record"
    out = ctypes.c_void_p()
    bad = [
        ibp.ibp_params(0, 32, 32, 0.95),        # L = 0
        ibp.ibp_params(6, 32, 32, 0.95),        # L not a multiple of 4
        ibp.ibp_params(64, 32, 48, 0.95),       # M not a multiple of W
        ibp.ibp_params(64, 32, 32, 0.5),        # T outside (0.5, 1]
        ibp.ibp_params(64, 32, 96 * 2, 0.95),   # M does not divide 8L
    ]
    for prm in bad:
        st = L.ibp_build_metadata(ctypes.byref(prm), None, 1, ctypes.byref(out), None)
        assert st == ibp.IBP_ERR_INVALID_ARG, prm
    prm = ibp.ibp_params(96, 96, 192, 0.95)  # W = 96: valid format, not on the GPU path
    assert L.ibp_build_metadata(ctypes.byref(prm), None, 1, ctypes.byref(out), None) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_meta_destroy(None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_check(None, None) == ibp.IBP_ERR_INVALID_ARG
    # packed-cache calls: a null handle or null offsets is rejected on the host
    assert L.ibp_packed_offsets(None, None, 0, None, None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_compress_packed(None, None, 1, None, None, 0, None, None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_decompress_packed(None, None, 0, None, None, 1, None, None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_gather_decompress_packed(None, None, 0, None, 1, None, None, 1, None, None) == \
        ibp.IBP_ERR_INVALID_ARG
    # header-in-GPU-memory calls
    assert L.ibp_compress_split(None, None, 1, None, None, None, None, None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_decompress_split(None, None, None, None, 1, None, None) == ibp.IBP_ERR_INVALID_ARG
    assert L.ibp_gather_decompress_split(None, None, 1, None, None, None, 1, None, None) == ibp.IBP_ERR_INVALID_ARG
