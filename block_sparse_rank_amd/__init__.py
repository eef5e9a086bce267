"""MI355X-native HSA + HKV forward: hand-written gfx950 HIP kernels behind a C ABI.

`block_sparse_rank_amd.hsakv` is the ctypes binding of libhsakv.so (see
include/hsakv.h); `block_sparse_rank_amd.build` compiles it in-tree.
"""
