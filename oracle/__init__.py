"""Plain fp64 CPU oracle for cache-aware block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library; inputs come from
the seeded generators in ``synth``.

Every function restates a computation from the two source pages:

* "WaveAlign: Cache-Aware Query-Row Scheduling for Sparse Attention in
  Long-Video Generation" (cited as *WaveAlign*): the block mask and row NNZ
  (§II-B, §II-C), column centering (§IV-C eq. (2)), the matrix-free centered
  subspace iteration (§IV-C-2, Algorithm 1), the polar ordering (§IV-C-1
  eq. (4)), the two-stage reordering (§IV-D, §IV-E, Algorithm 2) and the
  adaptive skip (§IV-E).
* "Sparse Attention for Video Generation Acceleration via Growing Sparsity and
  Reduced Search" (cited as *GSRS*): block-sparse attention with a row-wise
  log-sum-exp (§3 preliminaries), the two-phase block importance (§5.3,
  Appendix A.2), fully masked rows (note to Algorithm 2), Top-p selection
  (Algorithm 3) and the multi-step schedule of growing sparsity and reduced
  search (§4-5, Algorithm 4).
* The MinHash and banded-LSH row orders that WaveAlign's Table II compares
  against (``comparators``), from the published min-wise hashing and the banded
  locality-sensitive hashing of its signatures.

Floating point is fp64 throughout; bf16 inputs are widened exactly.  Where the
pages leave a step open the reading taken is stated in the function's
docstring.  Parity of the reorder *permutation* across implementations is
unpinned (near-ties of fp64 angles may order differently); what is pinned is
listed in each module.
"""

from .attention import (attention_distance, attention_entropy, masked_attention,  # noqa: F401
                        masked_attention_rows)
from .block_index import block_index  # noqa: F401
from .reorder import (  # noqa: F401
    ReorderParams,
    canonical_signs,
    centered_mask,
    mfcsi,
    polar_angles,
    reorder_head,
    reorder_rows,
    skip_decision,
    skip_statistics,
    stage1_order,
    stage2_order,
    wave_buckets,
)
from .gsrs import (  # noqa: F401
    block_importance,
    block_importance_from_probs,
    mask_recall,
    block_lse,
    cached_lse_scores,
    gsrs_schedule,
    topp_select,
)
from .permute import gather_blocks, scatter_blocks  # noqa: F401
from .comparators import (LSH_ROWS_PER_BAND, MINHASH_P, lsh_components,  # noqa: F401
                          lsh_order, lsh_order_head, minhash_order, minhash_order_head,
                          minhash_signatures)
