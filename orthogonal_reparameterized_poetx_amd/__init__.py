"""POET-X layer hot path on AMD Instinct MI355X (gfx950).

The compute lives in ``libpoetx.so`` (HIP kernels behind the C ABI declared in
``include/poetx.h``); this package is its thin Python binding, with PyTorch
tensors supplying device memory and streams.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    OP_BACKWARD,
    OP_BACKWARD_DQ,
    OP_BACKWARD_BLOCKS,
    OP_FORWARD,
    OP_FORWARD_BLOCKS,
    OP_MERGE,
    OP_MERGE_BLOCKS,
    POETX_ACCUMULATE_GRAD,
    POETX_W0_INT8,
    POETX_SEPARATE_BLOCK_PRODUCTS,
    POETX_BF16,
    POETX_F32,
    Blocks,
    BlockSet,
    ChainSet,
    Layer,
    PoetxError,
    build_cnp_workspace_bytes,
    build_workspace_bytes,
    chain_workspace_bytes,
    last_error,
    lib,
    make_blocks,
    make_workspace,
    poetx_adam_step,
    poetx_backward,
    poetx_backward_blocks,
    poetx_backward_blocks_dq,
    poetx_backward_blocks_dq_z2,
    poetx_dequantize_w0,
    poetx_build_block_sets,
    poetx_build_block_sets_cnp,
    poetx_build_blocks,
    poetx_chain_rule_sets,
    poetx_forward,
    poetx_forward_blocks,
    poetx_forward_blocks_noalloc,
    poetx_forward_blocks_z2,
    poetx_make_permutation,
    poetx_merge,
    poetx_merge_blocks,
    poetx_quantize_w0,
    timing_enable,
    timing_summary,
    w0_bytes,
    workspace_bytes,
)
from .layer import (PoetxLayer, build_layer_blocks, chain_rule_layers, merge_layers_sets,  # noqa: F401,E402
                    merge_sets_workspace_need)
