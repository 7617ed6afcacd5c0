"""MI355X (gfx950) hybrid compressed attention: DeepSeek-V4's CSA and HCA layers.

The compute lives in ``libcsa.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/csa.h``).  This module only marshals arguments: it
passes device pointers of torch tensors and the current HIP stream to the
library, and raises if the library reports an error.  There is no fallback:
importing without a built ``libcsa.so`` raises ``ImportError``.
"""
from __future__ import annotations

from .abi import (  # noqa: F401
    ACT_BF16, ACT_F32, CSAError, IDX_BF16, IDX_F32, IDX_MXFP4, KIND_CSA, KIND_HCA, KV_BF16, KV_F32, KV_FP8,
    OP_ATTENTION, OP_COMPRESS, OP_TOPK, Batch, LayerDesc, Sizes, abi_version, cache_append, compress_append,
    compress_kv, grouped_linear, hca_attention, index_scores, layer_sizes, lib, linear, prefix_blocks, prefix_bytes, prefix_state,
    sparse_mqa, topk_select, workspace_size,
)
from .layer import LayerState, make_batch  # noqa: F401
