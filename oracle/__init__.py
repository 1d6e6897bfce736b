"""fp64 CPU oracle for joint RoPE attention (test infrastructure).

This package is test infrastructure, not product code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path and never imports it; the only
module both sides use is the seeded input generator
``diffusion_transformer_joint_amd.inputs``, which holds no attention arithmetic.

What it computes (every function cites the passage it follows):
  * ``rope``       - multi-axis rotary position embedding in fp64;
  * ``softmax_attention`` - non-causal softmax attention over the whole joint sequence,
                     blocked over query rows, fp64;
  * ``e4m3``       - decoding of OCP 8-bit e4m3 ("e4m3fn") codes and
                     nearest-even rounding to them, from the format's definition;
  * ``fp8_requant`` - attention of the FP8 path with its second quantization
                     (rotated Q and K rounded to e4m3 again);
  * ``block_sparse`` - the tile-mask rules of threshold-sparse attention (the
                     score-bound rule with its error bound against dense
                     attention, and the pooled-score rule) and exact
                     attention over the kept tiles;
  * ``backward``   - gradients (dq, dk, dv) of joint RoPE attention and the
                     per-row log-sum-exp.

Parity status: every function here is pinned by tests in ``tests/test_oracle*.py``
(closed forms, brute force, independent formulations, invariants).  What no test can pin is whether these conventions (pair layout,
axis split, theta) are those of the real FLUX 3 model: no weights or model code
are available, and both sides of every comparison use the same convention.
"""
from .rope import rope_frequencies, rope_angles, apply_rope  # noqa: F401
from .softmax_attention import (softmax_rows, attention_from_scores, attention,  # noqa: F401
                        joint_rope_attention, joint_rope_attention_rows,
                        segment_local_rope_attention)
from .e4m3 import e4m3_decode, e4m3_table, dequantize, e4m3_round  # noqa: F401
from .fp8_requant import requantized_operands, fp8_requant_attention  # noqa: F401
from .inputs_fp64 import inputs_to_fp64  # noqa: F401
from .block_sparse import (tile_means, block_scores, block_mask, block_sparse_attention,  # noqa: F401
                           tile_score_maxima, bound_mask, skipped_mass, skip_mass_bound, dense_error_bound)
from .backward import rope_transpose, attention_lse, attention_backward  # noqa: F401
