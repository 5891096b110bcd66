"""CPU oracle for paged latent-KV MLA (test infrastructure only).

Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and it never
calls the HIP library.
"""
from .mla_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3_bits_to_f64,
    E4M3Pool,
    gather_latent_rows,
    visible_rows,
    mla_attention_loop,
    mla_attention_folded,
    mla_attention_rows,
    lse_merge,
    mla_attention_pages,
    tree_visible,
    mla_attention_tree,
    mla_attention_tree_loop,
    mla_attention_tree_rows,
    mla_attention_varlen,
    e4m3_quantize,
    mla_attention_nope,
    absorb_q,
    project_o,
    kv_append,
)
