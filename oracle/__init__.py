"""CPU oracle for the batched, rank-specialized LoRA-delta apply.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP library.

Every function is a plain, slow, obviously-correct restatement of what the
sources define (float64 unless stated, Python loops over tokens):

* ``segment_ref``  - stable grouping of tokens by adapter id
* ``shrink_ref``   - h = A_a x per token
* ``shrink_error_bound`` - the float32 accumulation bound of h (gamma_n form)
* ``apply_ref``    - y = y0 + s_a B_a (A_a x) per token
* ``base_fused_ref`` - y = W0 x + s_a B_a (A_a x) per token (the base layer with the branch)
* ``brute_force``  - the same in exact rational arithmetic, two association
                     orders, for tiny inputs
* ``bf16_round_ref`` - round-to-nearest-even onto bfloat16, used where a
                     floating-point result is compared bit for bit
* ``jd_apply_ref`` - the shared-basis apply y = y0 + s_a U_c Sigma_a V_c^T x
* ``jd_brute_force`` - the same in exact rational arithmetic, two orders
* ``uniform_ranks_ref``, ``spectral_ranks_ref`` - retained-rank allocation
                     (uniform ratio with a floor; spectral budget)
* ``retained_factors_ref``, ``tall_skinny_r_ref`` - retained factors by the
                     SVD of B A through thin QRs of B and A^T

Parity status: every function here is pinned by tests in
``tests/test_oracle.py`` (closed forms, invariants, brute force, library
routines, a hand-worked example); none is "parity unpinned".
"""
from .lora_ref import (  # noqa: F401
    apply_ref,
    base_fused_ref,
    bf16_round_ref,
    brute_force,
    segment_ref,
    shrink_ref,
    shrink_error_bound,
)
from .jd_ref import jd_apply_ref, jd_brute_force  # noqa: F401,E402
from .rank_ref import spectral_ranks_ref, uniform_ranks_ref  # noqa: F401,E402
from .rsvd_ref import retained_factors_ref, rsvd_ref, tall_skinny_r_ref  # noqa: F401,E402
