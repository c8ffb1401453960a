"""fp64 CPU oracle for one context-parallel rank's sparse-attention shard.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package
(``context_sparse_attention_amd``) imports, links or runs this code; only the
tests, the smoke check and the benchmark's CPU-baseline leg may.  The oracle
shares no code with the HIP path: it reads the same seeded inputs (from
``csa_inputs``) and computes every result from its own plain definitions.

Precision: every computation is float64 over the exact input values (bf16 and
fp32 inputs widen to float64 without loss).  Each function cites the passage it
follows; where the pages leave a step open, the reading taken is stated in the
docstring.  Sources (by page title):

* MoBA issue #34, "Question on Implementing Context Parallelism with MoBA
  Efficient Attention" - block selection from gating scores Q x K^T, top-k blocks.
* "Context parallel attention: exchange keys and merge softmax globally" -
  global positions decide the mask, packed sequences keep their boundaries,
  chunk summaries (m, l, z), merge by rescaling to the larger maximum, neutral
  summary for all-masked chunks, explicit convention for queries without keys.
* Megatron-LM issue #4878, "[Feature-request] Context Parallel support for
  DSAttention" - local queries against gathered keys with the causal diagonal
  shifted by the rank offset; top-k indices in global coordinates.
* Megatron-LM PR #3674, "[1/2] Enable DSA CP, THD with absorbed MLA" - an
  indexer picks the top-k key tokens of each query; packed THD masking;
  absorbed MLA (value = latent part of the key, up-projection after attention).
  The earlier PR description quoted on that page: the value up-projection is
  applied after sparse attention (``mla.v_up_proj``).

Parity status: every function here is pinned by a CPU test (tests/test_oracle_*),
except the input-generation conventions, which belong to ``csa_inputs``.
"""

from .layout import permitted_interval
from .moba import stream_blocks, pool_blocks, gate_candidates, gate_scores, select_blocks
from .dsa import indexer_logits_row, select_tokens_row, indexer_topk
from .attention import (
    NEUTRAL_M,
    slot_span,
    slot_keys,
    selected_keys,
    attend,
    attend_heads,
    attend_spans,
    shard_forward,
    summary,
    merge,
    finalize,
    merge_parts,
)
from .mla import v_up_proj
from .backward import shard_backward, loss

__all__ = [
    "permitted_interval",
    "stream_blocks",
    "pool_blocks",
    "gate_candidates",
    "gate_scores",
    "select_blocks",
    "indexer_logits_row",
    "select_tokens_row",
    "indexer_topk",
    "NEUTRAL_M",
    "slot_span",
    "slot_keys",
    "selected_keys",
    "attend",
    "attend_heads",
    "attend_spans",
    "shard_forward",
    "summary",
    "merge",
    "finalize",
    "merge_parts",
    "v_up_proj",
    "shard_backward",
    "loss",
]
