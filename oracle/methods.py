"""Direct definitions of each PEFT method, from its own raw parameters.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (page = the Scute paper, arXiv 2611.01089, as published on
paperpeel.com):
  * LoRA  -- §2 "The LoRA schedule": the update adds c·xAB to xW.
  * DoRA  -- §2 "The methods" and §5.1 "The Admission Compiler": each output
             column of W + cAB is rescaled to the learned magnitude m, so
             s = m ⊘ ‖W + cAB‖_c with the norm of each output column taken
             over d_in (appendix "Tensor parallelism").
  * (IA)3 -- §2 "The methods" and §3.1: a learned vector multiplies the
             projection's output (on the FFN, the up projection's output).
  * VeRA  -- §2 "The methods": one frozen pair A, B shared by every adapter;
             each adapter learns d inside the term and e after it.
  * OFT   -- §2 "The methods" and §3.1: the input is multiplied by a
             block-diagonal orthogonal R whose blocks are Cayley transforms
             of skew-symmetric matrices; the base layer is then unchanged.
  * SSF   -- §3.1 and Table 1: scale s and shift b on the output.
  * LoHa  -- §3.1 ("Other methods fit as well"): the update is built from
             products of small factors.  Reading: LoHa's own definition, the
             elementwise product of two low-rank products,
             ΔW = c · (A1 B1) ⊙ (A2 B2).
  * LoKr  -- same passage.  Reading: LoKr's own definition, a Kronecker
             product of a small matrix with a low-rank product,
             ΔW = c · (C ⊗ (A B)), C [p, q], A [d_in/p, r], B [r, d_out/q].
  * Stack -- §3.2 (paragraph "Stacking") and the appendix paragraph of that
             name: a second member applied at the same hook takes the first
             member's output in place of its own base output xW; its terms
             still read x.  Only the first member may transform the input
             (OFT), since a later member's base path is the previous output,
             not xW.

All arithmetic is numpy float64.  Matrices use the paper's row convention:
x [N, d_in], W [d_in, d_out], A [d_in, r], B [r, d_out].

Adapter records are plain dicts::

    {"method": "identity"}
    {"method": "lora", "A": A, "B": B, "c": c}
    {"method": "dora", "A": A, "B": B, "c": c, "m": m}
    {"method": "ia3",  "l": l}
    {"method": "vera", "d": d, "e": e, "c": c}      # + shared {"A": Av, "B": Bv}
    {"method": "oft",  "Q": Q}                       # Q: [d_in / b, b, b] skew
    {"method": "ssf",  "s": s, "b": b}
    {"method": "loha", "A": A1, "B": B1, "A2": A2, "B2": B2, "c": c}
    {"method": "lokr", "C": C, "A": A, "B": B, "c": c}
    {"method": "stack", "members": [rec1, rec2, ...]}   # applied in order
"""
import numpy as np

METHODS = ("identity", "lora", "dora", "ia3", "vera", "oft", "ssf", "loha", "lokr", "stack")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def cayley(Q):
    """Cayley transform of one skew-symmetric block: R = (I + Q)(I - Q)^-1.

    Page: §2 "The methods" (OFT blocks are Cayley transforms of
    skew-symmetric matrices) and the appendix "Training" (the library's
    default Cayley form).  The pages do not print the formula; this is the
    textbook Cayley map, with an exact inverse (no truncated series).  The
    other common convention, (I - Q)(I + Q)^-1, equals the transpose of this
    one.
    """
    Q = _f64(Q)
    eye = np.eye(Q.shape[0])
    return (eye + Q) @ np.linalg.inv(eye - Q)


def oft_rotation(Q):
    """Block-diagonal R from skew blocks Q [n_blocks, b, b] (§2, §3.1)."""
    Q = _f64(Q)
    nb, b, _ = Q.shape
    R = np.zeros((nb * b, nb * b))
    for j in range(nb):
        R[j * b:(j + 1) * b, j * b:(j + 1) * b] = cayley(Q[j])
    return R


def dora_column_norm(W, A, B, c):
    """‖W + cAB‖_c: for each output column, the 2-norm over d_in.

    Page: §5.1 (s = m ⊘ ‖W + cAB‖_c, "the norm of each output column") and
    the appendix "Tensor parallelism" (taken over d_in for each output
    column).
    """
    Wp = _f64(W) + float(c) * (_f64(A) @ _f64(B))
    return np.sqrt(np.sum(Wp * Wp, axis=0))


def dora_scale(W, A, B, c, m):
    """DoRA's output scale s = m ⊘ ‖W + cAB‖_c (§5.1)."""
    return _f64(m) / dora_column_norm(W, A, B, c)


def base_forward(x, W):
    """h = xW, the shared base GEMM (§2 "The LoRA schedule")."""
    return _f64(x) @ _f64(W)


def direct_forward(x, W, adapter, shared=None):
    """Output of one adapted projection for rows x, by the method's own
    definition from its raw parameters (module docstring gives the source
    of each branch).  ``shared`` holds VeRA's frozen pair {"A", "B"}."""
    x = _f64(x)
    W = _f64(W)
    meth = adapter["method"]
    if meth == "identity":
        return x @ W
    if meth == "lora":
        A, B, c = _f64(adapter["A"]), _f64(adapter["B"]), float(adapter["c"])
        return x @ W + c * ((x @ A) @ B)
    if meth == "dora":
        A, B, c = _f64(adapter["A"]), _f64(adapter["B"]), float(adapter["c"])
        Wp = W + c * (A @ B)                      # the adapted weight
        norm = np.sqrt(np.sum(Wp * Wp, axis=0))   # per output column
        return (x @ Wp) * (_f64(adapter["m"]) / norm)
    if meth == "ia3":
        return (x @ W) * _f64(adapter["l"])
    if meth == "ssf":
        return (x @ W) * _f64(adapter["s"]) + _f64(adapter["b"])
    if meth == "vera":
        if shared is None:
            raise ValueError("VeRA needs the shared pair")
        Av, Bv = _f64(shared["A"]), _f64(shared["B"])
        c = float(adapter.get("c", 1.0))
        d, e = _f64(adapter["d"]), _f64(adapter["e"])
        return x @ W + c * ((((x @ Av) * d) @ Bv) * e)
    if meth == "oft":
        R = oft_rotation(adapter["Q"])
        return (x @ R) @ W
    if meth in ("loha", "lokr"):
        return x @ W + x @ product_update(adapter)
    if meth == "stack":
        members = adapter["members"]
        y = direct_forward(x, W, members[0], shared)
        for mem in members[1:]:
            y = applied_to(y, x, W, mem, shared)
        return y
    raise ValueError("unknown method %r" % (meth,))


def product_update(adapter):
    """ΔW [d_in, d_out] of LoHa or LoKr, formed densely from its factors."""
    c = float(adapter["c"])
    if adapter["method"] == "loha":
        return c * ((_f64(adapter["A"]) @ _f64(adapter["B"])) * (_f64(adapter["A2"]) @ _f64(adapter["B2"])))
    if adapter["method"] == "lokr":
        return c * np.kron(_f64(adapter["C"]), _f64(adapter["A"]) @ _f64(adapter["B"]))
    raise ValueError("not a product method: %r" % (adapter["method"],))


def applied_to(y, x, W, adapter, shared=None):
    """A member applied at a hook whose base output is already y (the
    previous member's output) instead of xW: each method's definition with
    xW replaced by y.  DoRA's magnitude still rescales the columns of its
    own adapted weight W + cAB, so its scale comes from W as on its own."""
    y = _f64(y)
    x = _f64(x)
    meth = adapter["method"]
    if meth == "identity":
        return y.copy()
    if meth == "lora":
        A, B, c = _f64(adapter["A"]), _f64(adapter["B"]), float(adapter["c"])
        return y + c * ((x @ A) @ B)
    if meth == "dora":
        A, B, c = _f64(adapter["A"]), _f64(adapter["B"]), float(adapter["c"])
        return (y + c * ((x @ A) @ B)) * dora_scale(W, A, B, c, adapter["m"])
    if meth == "ia3":
        return y * _f64(adapter["l"])
    if meth == "ssf":
        return y * _f64(adapter["s"]) + _f64(adapter["b"])
    if meth == "vera":
        Av, Bv = _f64(shared["A"]), _f64(shared["B"])
        c = float(adapter.get("c", 1.0))
        return y + c * ((((x @ Av) * _f64(adapter["d"])) @ Bv) * _f64(adapter["e"]))
    if meth in ("loha", "lokr"):
        return y + x @ product_update(adapter)
    if meth == "oft":
        raise ValueError("only the first member of a stack may transform the input")
    raise ValueError("unknown method %r" % (meth,))


def input_transform(adapter, d_in):
    """R of the adapter (identity unless OFT), used for the base output
    h = (xR)W that the parity bound is measured against."""
    if adapter["method"] == "oft":
        return oft_rotation(adapter["Q"])
    if adapter["method"] == "stack":
        return input_transform(adapter["members"][0], d_in)
    return np.eye(d_in)
