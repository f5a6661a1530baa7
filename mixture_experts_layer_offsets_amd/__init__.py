"""MI355X-native MoE layer (forward + backward): Python face of libmoe.

``_lib`` exposes the C entry points of ``include/moe.h`` under the same names;
``MoeLayer`` owns the caller-side buffers (workspace, saved context, packed
weights) as torch tensors and calls those entry points.  All computation is in
libmoe's HIP kernels.
"""
from ._lib import (MOE_BF16, MOE_ERR_DEVICE_TIMEOUT, MOE_MXFP8, MOE_MXFP8_W4,  # noqa: F401
                   MOE_MXFP8_W6, MOE_MXFP8_W6E3M2, MOE_OK, MoeError,
                   MOE_SCHED_PERSISTENT, MOE_SCHED_PIPELINED, MOE_SCHED_STAGED,
                   MoeSched, Shape, WEIGHT_FORMAT, load,
                   moe_combine, moe_decode_fwd, moe_dispatch, moe_expert_ffn, moe_layer_bwd, moe_layer_fwd,
                   moe_layout, moe_layout_noalloc, moe_packed_pointers, moe_packed_weight_bytes,
                   moe_prepare_weights,
                   moe_read_status,
                   moe_route, moe_router_logits, moe_saved_bytes, moe_saved_pointers,
                   moe_strerror, moe_workspace_bytes, moe_workspace_pointers)
from .layer import MoeLayer  # noqa: F401
