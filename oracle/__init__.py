"""CPU float64 oracle for split-KV MLA decode with the LSE combine.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``split_kv_mla_amd/``.

See ``oracle/mla_oracle.py`` for the definitions and their sources.
"""

from .mla_oracle import (  # noqa: F401
    D_QK,
    D_V,
    bf16_bits_to_f64,
    fp8_e4m3_to_f64,
    kv_rows_to_f64,
    row_length,
    shard_of_token,
    shard_token_sets,
    gather_rows,
    attention_row,
    mla_decode_oracle,
    lse_combine_oracle,
    merge_states_oracle,
    padding_row_mask,
    local_index_of_token,
    chunked_context_alignment,
    align_chunked_context_workspace,
    context_chunk_plan,
    gather_context_chunk_oracle,
)
