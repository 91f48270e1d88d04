"""MI355X-native unified block-sparse attention with hierarchical, query-aware
KV page selection.

The compute path is the HIP library liblsa.so (C ABI in include/lsa.h);
`lsa` is its ctypes binding and `workloads` the seeded synthetic input
generators.  Build with `python -m block_sparse_attention_logical_amd.build`.
"""
from . import lsa  # noqa: F401
from .lsa import (  # noqa: F401
    BF16, F32, INT4, RETRIEVAL, STREAMING, Heads, KVPool, LsaError, build_page_stats, decode_workspace,
    page_stats_bytes, select_pages, select_pages_workspace, sparse_decode_attn, sparse_prefill_attn,
)
