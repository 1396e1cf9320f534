"""MI355X (gfx950) paged MLA decode over a context-sharded KV cache.

The compute lives in libmla_dcp.so (HIP kernels behind the C ABI of
include/mla_dcp.h); ``_lib`` is its ctypes binding and ``step`` runs one
sharded decode step (metadata, partial decode per shard, merge).
"""
from ._lib import (LSE_BASE_2, LSE_BASE_E, MlaError, load, mla_build_shard_metadata,
                   mla_decode_partial, mla_decode_workspace_bytes, mla_merge_partials)
