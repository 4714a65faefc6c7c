"""CPU float64 oracle for the batched multi-adapter layer in normal form.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this
module.  It may be imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py`` -- nowhere else.  The HIP
path never calls it and it never calls the HIP path; the two share no code.

What it computes (Scute paper, arXiv 2611.01089, "§3.1 The Normal Form",
eq. (1) and Table 1): each row of a batch belongs to one tenant, and the
tenant's adapter is applied to the shared base weight W by the plain
definition of its PEFT method (LoRA, DoRA, (IA)3, VeRA, OFT, SSF, LoHa,
LoKr, or a stack of members applied in order), evaluated from the adapter's
own raw parameters in numpy float64.  A second path
evaluates eq. (1) literally from the adapter's slots, unfolded and folded.

Conventions (the paper's): rows are tokens, ``x`` is ``[N, d_in]``, the
math-layout base weight ``W`` is ``[d_in, d_out]`` (the transpose of an
``nn.Linear`` weight), ``A`` is ``[d_in, r]`` and ``B`` is ``[r, d_out]``.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
identities the pages state, hand-derived values in ``tests/golden/`` and a
pure-Python brute force on tiny inputs.  No function here is "parity
unpinned".
"""
from .methods import (  # noqa: F401
    METHODS,
    applied_to,
    product_update,
    cayley,
    oft_rotation,
    dora_column_norm,
    dora_scale,
    direct_forward,
    base_forward,
)
from .normal_form import (  # noqa: F401
    SLOT_NAMES,
    unfolded_slots,
    fold,
    normal_form_eval,
    member_table,
    fold_rule,
    stack,
    expand_product,
)
from .layer import layer_forward, plan, parity_metrics  # noqa: F401
