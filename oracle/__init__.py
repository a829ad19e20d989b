"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The HIP library
(``io_aware_exact_03_amd``) never imports it and shares no code with it; the
only module both sides use is the seeded input generator ``fa_synth``, which
holds none of the method's arithmetic.

Pages cited in this package (by title and section; the text is theirs, the code
is ours):

* [essay]  "Flash Attention: IO-awareness principle" (hrletsgo.me documents),
  sections "Standard Attention's real bottleneck", "Tiling", "Recomputation",
  the section "FA2/FA3" (FP8 mode, oracle/fp8.py),
  and the sections on serving (grouped-query attention, oracle/gqa.py;
  decoding, oracle/decode.py) and on PagedAttention and chunked prefill
  (oracle/chunk.py).
* [lesson] "Flash Attention -- five lessons converging into 80 lines",
  CUDA training lesson 06 (brianyu43.github.io), sections "Results",
  "Lesson 1", "LLM-serving translation" (decode: one query per head).
* [triton] "Triton 06: Flash Attention v2" (wonbeomjang.kr), sections
  "Improvement 1: un-scaled accumulation", "Improvement 2: exp -> exp2",
  "Improvement 3: causal mask 2-stage", "Backward", "Forward/Backward flow".
* [review] "Paper review: FlashAttention: Fast and Memory-Efficient Exact
  Attention with IO-Awareness" (osehyeon.github.io), Algorithm 0, the softmax
  decomposition under "Tiling", Algorithm 1.

Every function here is pinned by tests under ``tests/test_oracle.py`` against
closed forms, invariants, finite differences, brute force on tiny inputs,
independent library routines, and the worked numbers the pages print.
"""
from .attention import (  # noqa: F401
    attn_fwd,
    attn_bwd,
    attn_fwd_rows,
    attn_fwd_bruteforce,
    attn_bwd_bruteforce,
    online_fa1,
    online_fa2,
    fa1_block_sizes,
    causal_stage_ranges,
    loss,
)
from .gqa import attn_bwd_gqa, attn_fwd_gqa, attn_fwd_rows_gqa  # noqa: F401
from .fp8 import (  # noqa: F401
    attn_fwd_fp8, attn_fwd_fp8_model, attn_fwd_fp8_rows, dequantize, e4m3_decode, e4m3_round, p_rounding_bound)
from .chunk import attn_fwd_chunk, attn_fwd_chunk_rows  # noqa: F401
from .decode import attn_decode, decode_partials, decode_split_merge, merge_partials, split_bounds  # noqa: F401
