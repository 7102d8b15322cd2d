"""MI355X (gfx950) routed-expert MXFP4 MoE layer.

Python binding of the C ABI in include/moe_mxfp4.h.  Every function here
only marshals torch tensors into pointers, sizes and the current HIP stream
and calls the library; all arithmetic runs in the HIP kernels.  There is no
CPU fallback: if libmoe_mxfp4.so is missing or the device is not gfx950 the
calls raise.

One layer (the routed experts of a Kimi K3 layer: 16 experts picked per
token, MXFP4 weights, SwiGLU FFN, weighted combine):

    logits = router_logits(x, w_router)      # the projection before the path
    ids, w = route_topk(logits, k)
    grp = group_rows(ids, E, workspace)
    y_rows = expert_ffn_mxfp4(x, k, pool, grp, workspace)
    out = combine(y_rows, w, grp.row_pos)

One token at a time (decode, the layer stack), route_group_one replaces the
first two calls and combine_rms_bf16 fuses the combine with the RMS rescale
that feeds the next layer.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    MoeError,
    ExpertPool,
    Grouping,
    MoeWeights,
    combine,
    combine_rms_bf16,
    decode_layer_mxfp4,
    decode_layer_mxfp4_noalloc,
    decode_layer_rms_mxfp4,
    expert_ffn_combine_mxfp4,
    expert_ffn_mxfp4,
    group_rows,
    lib,
    rms_rescale_bf16,
    route_group_one,
    route_topk,
    router_logits,
    status_string,
    workspace_bytes,
    MAX_EXPERTS,
    MAX_TOPK,
    MAX_DIM,
)
