"""CPU oracle of the sparse-decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code in float64.  Only the tests, the
smoke check and the bench's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and shares no code,
header, table or helper with it.

Sources.  The four web pages about SparseEngine (arXiv:2609.39068) fix what
each method does, one sentence each; every function below names the page and
section it follows.  Short names used in the docstrings:

  [jetabc]  jetabc.cn, "长程 agent 把显存撑爆以后：哈工大 SparseEngine 为什么要从零重建推理引擎"
  [tokendh] tokendh.com news f00df0ef4a, the SparseEngine explainer
  [netics]  Netics blog, "SparseEngine 统一接入十五种稀疏注意力"
  [aifeeds] ai-feeds.com paper digest, "SparseEngine：稀疏优先推理引擎"

Where the pages leave a step open, the reading taken is stated in the
function's docstring (and collected in the design notes).

Decisions (which page, which token) are taken on float32-rounded scores, the
precision the GPU kernels score in; everything else stays float64.

Pins: every function here is checked by `tests/test_oracle_pins.py` against
library routines, closed forms, invariants and brute force.  Fidelity to the
*original* Quest, SnapKV, H2O and OmniKV papers beyond what the pages state is
parity unpinned (see `UNPINNED` below).
"""
from .selection import top_k_ascending, argmin_lower, boundary_gap, argmin_gap  # noqa: F401
from .quest import page_meta, quest_bounds, quest_select  # noqa: F401
from .attention import view_tokens, decode_attention, unit_attention  # noqa: F401
from .snapkv import snapkv_votes, snapkv_pool, snapkv_keep, snapkv_compact  # noqa: F401
from .h2o import h2o_accumulate_evict, h2o_step  # noqa: F401
from .omnikv import omnikv_scores, omnikv_select, omnikv_layer_views  # noqa: F401
from .variants import streaming_kept, streaming_view, pyramid_budgets  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, quantize_rows, dequantize_rows  # noqa: F401

UNPINNED = (
    "Group aggregation of the Quest bound (max over the group's heads), "
    "whether the SnapKV window counts in its budget, the SnapKV softmax denominator, "
    "H2O's step order and candidate set, and OmniKV's per-KV-head selection are readings "
    "of pages that state each method in one sentence; nothing on the pages confirms them.  "
    "StreamingLLM (first and last positions) and PyramidKV (arithmetic per-layer budgets "
    "around SnapKV) are only named on the pages; their forms here are readings too."
)
