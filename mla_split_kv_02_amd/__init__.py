"""Python binding of libmla_decode.so (absorbed-MLA split-KV decode for MI355X).

Argument marshalling only: every step of the decode runs in the HIP kernels behind the
C ABI declared in ``include/mla_decode.h``.  torch provides device memory and the
current HIP stream.  Importing this package does not need a GPU; calling a compute
function without the built library, or without a GPU, raises.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MLA_ERR_HIP,
    MLA_ERR_INVALID_ARG,
    MLA_ERR_SCRATCH_LIMIT,
    MLA_ERR_UNSUPPORTED,
    MLA_ERR_WORKSPACE_TOO_SMALL,
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3,
    MLA_KV_FP8_E4M3_QFP8,
    MLA_KV_NVFP4,
    MLA_NOALLOC_SCRATCH_BYTES,
    MLA_OK,
    EXPORTED_SYMBOLS,
    MlaError,
    PagedCall,
    decode_splitkv,
    device_num_cus,
    kv_append,
    lib,
    paged_decode,
    paged_decode_noalloc,
    paged_decode_splits,
    paged_splits_workspace_bytes,
    paged_workspace,
    paged_workspace_bytes,
    plan_contig,
    plan_paged,
    plan_paged_splits,
    splitkv_combine,
    status_string,
)
