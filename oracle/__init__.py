"""CPU reference oracle for the LoGRA sketch-accumulate / RowAdam / merge path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import this
package.  The only callers are ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP library:
the sign generator, the sketch, RowAdam, the merge and the predicted-KL
step size are all written again here, in float64, from the definitions on the pages.

Source pages (cited by title and section / equation only):
  [LoGRA]  "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
           Sketches" (arXiv 2610.06647v2), full paper text.
  [Philox] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
           1, 2, 3", SC'11 (published definition of Philox4x64-10).
"""

from .logra_oracle import (  # noqa: F401
    MASK64,
    PHILOX_BLOCK_BITS,
    philox4x64_10,
    sign_bits,
    sign_matrix,
    rademacher_projection,
    gaussian_normals,
    gaussian_projection,
    GAUSS_PER_BLOCK,
    bf16_bits_to_f64,
    round_to_bf16,
    f64_to_bf16_bits,
    dense_gradient,
    sketch_from_gradient,
    project_inputs,
    sketch_accumulate,
    low_rank_expand,
    merge_update,
    rowadam_scale,
    reconstruction_cosine,
    sketch_accumulate_rounded_projection,
    sketch_projected_first,
)
from .predicted_kl import (  # noqa: F401
    token_probabilities,
    score_rate_variance,
    predicted_kl,
    policy_kl_along,
    kl_step_scale,
    kl_budget,
    effective_budget,
)
