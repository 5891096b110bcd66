"""MI355X (gfx950) paged latent-KV MLA: decode with the draft axis folded into the
head axis, and chunked prefill over a long cached prefix.

The computation lives in libmla.so (hand-written HIP kernels behind the C ABI in
include/mla.h); the functions here marshal torch device tensors into that ABI.
Importing this package loads nothing; the library is opened on first use.
"""
from ._binding import (  # noqa: F401
    BoundDecode,
    bound_absorb_q,
    bound_project_o,
    absorb_q,
    project_o,
    bound_kv_append,
    MLAError,
    LIB_PATH,
    auto_partitions,
    decode,
    decode_combine,
    decode_e4m3,
    decode_nope,
    decode_noalloc,
    decode_single_pass,
    decode_single_pass_e4m3,
    decode_splitkv,
    decode_splitkv_placement,
    decode_splitkv_timeline,
    decode_splitkv_e4m3,
    decode_tree,
    decode_varlen,
    header_functions,
    kv_append,
    lib,
    new_workspace,
    prefill_with_prefix,
    read_error_flags,
    status_string,
    workspace_bytes,
    workspace_size,
)
