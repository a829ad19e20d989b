"""MI355X (gfx950) exact attention: a fused FlashAttention-style forward and
backward plus a naive three-kernel baseline, all hand-written HIP behind the
C ABI of include/fa.h.  torch is used only for device memory and streams."""
from .ops import (  # noqa: F401
    DTYPE_CODES, ceiling_copy, ceiling_mfma, ceiling_mfma_flops, ceiling_mix, ceiling_mix_flops, ceiling_read, ceiling_valu, bwd, bwd_gqa, bwd_stage, causal_stages, decode, decode_noalloc, decode_pieces, decode_plan, decode_workspace_bytes,
    fa1_state, fa1_workspace_bytes, fwd, fwd_chunk, fwd_fa1, fwd_fp8, fwd_gqa, fwd_tile, kv_head, naive_fwd,
    naive_workspace_bytes)
