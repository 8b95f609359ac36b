"""MI355X-native Invariant Bit Packing (IBP): gfx950 HIP kernels behind a C ABI.

The binding to the C ABI lives in ``lossless_tensor_compression_ibp_amd.ibp``
and the seeded workload generators in ``.workloads``; neither is imported
here so that importing the package never touches a GPU.
"""
