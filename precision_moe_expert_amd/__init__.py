"""MI355X (gfx950) low-precision MoE expert forward.

The compute lives in libmoe_lp.so (HIP kernels behind the C ABI of
include/moe_lp.h); `binding` marshals torch tensors into it.  `synth` holds the
seeded synthetic input generators.
"""
from . import binding  # noqa: F401
from .binding import (FMT_FP8, FMT_FP8_POW2, FMT_INT4, FMT_MXFP4, FMT_NVFP4, WL_KBLOCKED, WL_ROWS,  # noqa: F401
                      MoeError, combine, expert_backward, expert_forward, expert_forward_materialized,
                      expert_forward_noalloc, lm_head_logprob, make_layer, pack_weights_kblocked,
                      prepare_backward_weights, route_permute, workspace_bytes)
