"""MI355X (gfx950) exact attention: a fused FlashAttention-style forward and
backward plus a naive three-kernel baseline, all hand-written HIP behind the
C ABI of include/fa.h.  torch is used only for device memory and streams."""
from .ops import fwd, bwd, bwd_stage, naive_fwd, naive_workspace_bytes, causal_stages, fwd_tile, DTYPE_CODES  # noqa: F401
