"""fp64 CPU oracle for one window step of WeDLM's Streaming Parallel Decoding.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it. It shares no code with the HIP
library (no kernels, headers, helpers, tables or layout code); the seeded input
generators are the only thing both sides consume, and they hold none of the
method's arithmetic.

Sources (the pages this oracle is written from):
  * "WeDLM" paper summary at hyper.ai, section "Method": the window step
    (reorder filled before masks with logical positions kept, a causal forward
    over the window conditioned on the persistent KV cache, commit of the
    leftmost contiguous filled run, refill with masks, distance-penalised
    entropy selection; the forward pass's predictions come from a projection
    of each slot's hidden state onto the vocabulary).
  * WeDLM review at sai.science, sections "Summary", "Weaknesses",
    "Reproducibility & code": RoPE keeps logical positions; the score equation
    is missing from the text; the entropy-threshold flag and the one-by-one
    mode.
  * mlsanity.com page on WeDLM, "Builds on": RoFormer (RoPE), PagedAttention,
    FlashAttention as prior art.

Everything is computed in float64 with no intermediate rounding. Integer
outputs are exact. The readings adopted where the pages are silent are listed
in each function's docstring.

Parity status:
  * reorder, RoPE, attention, entropy, vocabulary projection, dual-stream
    attention: pinned (tests/test_oracle_*.py).
  * the select fallback (a step where no mask slot clears the threshold fills
    the single lowest-score mask slot): parity unpinned. The pages do not say
    what happens then; the rule is a reading, exercised by hand-worked cases
    only.
"""

from .reorder import topological_reorder
from .rope import rope_frequencies, rope_rotate
from .attention import window_attention_reordered, window_attention_masked, visible_mask
from .entropy import vocab_entropy_argmax
from .select import select_slots
from .commit import commit_and_refill, cache_slot_of, commit_count
from .lm_head import vocab_projection, lm_head_select
from .dual_stream import dual_stream_attention
from .step import window_step, stream_loop

__all__ = [
    "topological_reorder",
    "rope_frequencies",
    "rope_rotate",
    "window_attention_reordered",
    "window_attention_masked",
    "visible_mask",
    "vocab_entropy_argmax",
    "select_slots",
    "commit_and_refill",
    "cache_slot_of",
    "commit_count",
    "vocab_projection",
    "dual_stream_attention",
    "lm_head_select",
    "window_step",
    "stream_loop",
]
