"""MI355X (gfx950) sequence-mixer forward library.

Gaussian Mixture Attention (causal and bidirectional), chunkwise decayed linear
attention, the gated delta rule and the curvature-conditioned-query read over
either write rule (with a carried state and
one-token decode steps for the causal forms), as hand-written HIP kernels
behind a C ABI (include/linmix.h). This package holds the ctypes binding
(`binding`), the build script (`build`) and the seeded input generator
(`inputs`). The library loads on the first call.
"""
from .binding import (LinmixError, ccq_decode_step, linattn_backward_workspace_bytes, linattn_chunk_backward,
                      linattn_chunk_backward_state,
                      gma_backward, gma_backward_workspace_bytes, ccq_backward, ccq_backward_workspace_bytes, ccq_forward, ccq_forward_state, ccq_state_size,
                      ccq_workspace_bytes, gma_decode_step, gma_forward, gma_forward_state, gma_state_size,
                      gma_workspace_bytes, linattn_chunk_forward, linattn_chunk_forward_state, linattn_decode_step,
                      linattn_state_size, linattn_vec_decode_step, linattn_vec_forward,
                      linattn_vec_forward_state, linattn_vec_workspace_bytes,
                      linattn_workspace_bytes, deltanet_chunk_forward, deltanet_forward_state,
                      deltanet_workspace_bytes, ccq_deltanet_forward, ccq_deltanet_forward_state,
                      ccq_deltanet_workspace_bytes)

__all__ = ["gma_forward", "linattn_chunk_forward", "ccq_forward", "gma_workspace_bytes",
           "linattn_workspace_bytes", "ccq_workspace_bytes", "gma_forward_state", "linattn_chunk_forward_state",
           "ccq_forward_state", "gma_decode_step", "linattn_decode_step", "ccq_decode_step", "gma_state_size",
           "linattn_state_size", "ccq_state_size", "linattn_vec_forward",
           "linattn_vec_workspace_bytes", "linattn_vec_forward_state", "linattn_vec_decode_step", "linattn_chunk_backward", "linattn_chunk_backward_state", "gma_backward", "gma_backward_workspace_bytes", "ccq_backward",
           "ccq_backward_workspace_bytes",
           "linattn_backward_workspace_bytes", "deltanet_chunk_forward", "deltanet_forward_state",
           "deltanet_workspace_bytes", "ccq_deltanet_forward", "ccq_deltanet_forward_state",
           "ccq_deltanet_workspace_bytes", "LinmixError"]
