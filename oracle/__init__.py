"""Plain fp64 CPU oracle for banded balanced Sinkhorn attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
this package imports nothing from the product path.

Source of the method: the arXiv paper "Block-Wise Differentiable Sinkhorn
Attention: Tail-Refinement Gradients with a Gap-Aware Dustbin Bridge"
(arXiv 2605.08123), as summarised on the pages cited in each docstring:

* abstract (dzcademia.com and searcharxiv.com listings)
* technical summary, German (gist.science/de), "Technische Zusammenfassung" §1-§5
* technical summary, French (gist.science/fr), "Résumé Technique" §1-§5
* AI-extracted summary (atlas.scime.ai), sections Approach / Key results /
  Limitations / Builds on

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, an independent multiplicative Sinkhorn, dense
torch autograd, central finite differences, marginal and orbit invariants).
The pages print no worked numeric example, so no value is pinned to a printed
number from the pages themselves.
"""

from .sinkhorn_band import (  # noqa: F401
    band_scores,
    row_update,
    col_update,
    forward,
    forward_from_base,
    vjp_one_reference,
    vjp_direct_four,
    vjp_tail,
    vjp_tail_one_reference,
    vjp_full,
    tail_remainder,
    select_tail_depth,
    staircase_plan,
    dustbin_block_forward,
    dustbin_block_vjp,
    dependency_radius,
    sampled_rows,
    row_range,
    BandProblem,
)
from .training import (  # noqa: F401
    TrainConfig,
    reconstruction_step,
    reconstruction_loss,
)
from .contraction import (  # noqa: F401
    block_layout,
    block_diameters,
    contraction_coefficients,
)
