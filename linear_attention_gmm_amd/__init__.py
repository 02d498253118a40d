"""MI355X (gfx950) sequence-mixer forward library.

Gaussian Mixture Attention (causal and bidirectional), chunkwise decayed linear
attention and the curvature-conditioned-query read, as hand-written HIP kernels
behind a C ABI (include/linmix.h). This package holds the ctypes binding
(`binding`), the build script (`build`) and the seeded input generator
(`inputs`). The library loads on the first call.
"""
from .binding import (LinmixError, ccq_forward, ccq_workspace_bytes, gma_forward, gma_workspace_bytes,
                      linattn_chunk_forward, linattn_workspace_bytes)

__all__ = ["gma_forward", "linattn_chunk_forward", "ccq_forward", "gma_workspace_bytes",
           "linattn_workspace_bytes", "ccq_workspace_bytes", "LinmixError"]
