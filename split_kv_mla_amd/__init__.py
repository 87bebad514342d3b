"""Split-KV MLA decode with the exp2 LSE combine on MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/mla_split_kv.h`` (``libmla_split_kv.so``, built in-tree by
``split_kv_mla_amd/build.py``); this package is its ctypes binding.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    MlaDecodeArgs,
    MlaError,
    MlaGatherArgs,
    decode_args,
    load_library,
    mla_align_chunked_context_workspace,
    mla_chunked_context_alignment,
    mla_context_chunk_plan,
    mla_gather_context_chunk,
    mla_device_faults,
    mla_lse_combine,
    mla_merge_states,
    mla_plan_capacity,
    mla_shard_decode_partial,
    mla_split_decode,
    mla_split_decode_static,
    mla_workspace_bytes,
    new_workspace,
)
