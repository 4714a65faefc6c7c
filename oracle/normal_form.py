"""The normal form, eq. (1), its slots, the fold rule and stacking.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page: the Scute paper (arXiv 2611.01089).
  * §3.1, eq. (1):
      F_a(x) = ((xR)W) ⊙ s + b + Σ_k c_k (((x A_k) ⊙ d_k) B_k ⊙ e_k)
    Six slots hold an adapter's own tensors: R, s, b on the base side and
    c_k, d_k, e_k on each term.  Unused slots hold the identity
    (I, 1, 0, 1, 1, 1).
  * Table 1: which matrices each method owns, its folds, its live slots.
  * §3.2 and the appendix "Folds" / "Proposition A1, the 'if' direction":
    c_k folds when any of A_k, d_k, B_k, e_k is owned; d_k folds when A_k or
    B_k is owned; e_k folds when B_k is owned; s, b and R never fold.  The
    identities used are (xA)⊙d = x(A diag d), ((xA)⊙d)B = (xA)(diag(d)B),
    (VB)⊙e = V(B diag e) and cA = (cA)·1.
  * Appendix "Stacking": F2 applied to the output of F1 is again a member,
    with scale s1⊙s2, shift b1⊙s2 + b2 and F1's terms scaled by s2 through e.
"""
import numpy as np

from .methods import _f64, dora_scale, oft_rotation

# Slots of eq. (1): base side R, s, b; per term c, d, e.
SLOT_NAMES = ("R", "s", "b", "c", "d", "e")


def unfolded_slots(adapter, W, shared=None):
    """Write an adapter in normal form with nothing folded (§3.1, Table 1,
    §5.1).  Returns {"R", "s", "b", "terms", "owned"}; a slot that is the
    identity is None.  Each term is {"c", "A", "d", "B", "e"}; "owned" names
    the tensors the adapter owns ("A", "B" of its term, "d", "e", "R")."""
    W = _f64(W)
    d_in, d_out = W.shape
    meth = adapter["method"]
    out = {"R": None, "s": None, "b": None, "terms": [], "owned": set()}
    if meth == "identity":
        return out
    if meth == "lora":
        out["terms"].append({"c": float(adapter["c"]), "A": _f64(adapter["A"]),
                             "d": None, "B": _f64(adapter["B"]), "e": None})
        out["owned"] = {"A", "B"}
        return out
    if meth == "dora":
        # §5.1: s = m ⊘ ‖W + cAB‖_c; the term carries the same scale as its
        # outer vector e, so F = (xW)⊙s + c((xA)B)⊙s.
        s = dora_scale(W, adapter["A"], adapter["B"], adapter["c"], adapter["m"])
        out["s"] = s
        out["terms"].append({"c": float(adapter["c"]), "A": _f64(adapter["A"]),
                             "d": None, "B": _f64(adapter["B"]), "e": s.copy()})
        out["owned"] = {"A", "B"}
        return out
    if meth == "ia3":
        out["s"] = _f64(adapter["l"])
        return out
    if meth == "ssf":
        out["s"] = _f64(adapter["s"])
        out["b"] = _f64(adapter["b"])
        return out
    if meth == "vera":
        out["terms"].append({"c": float(adapter.get("c", 1.0)), "A": _f64(shared["A"]),
                             "d": _f64(adapter["d"]), "B": _f64(shared["B"]),
                             "e": _f64(adapter["e"])})
        out["owned"] = {"d", "e"}
        return out
    if meth == "oft":
        out["R"] = oft_rotation(adapter["Q"])
        out["owned"] = {"R"}
        return out
    if meth in ("loha", "lokr"):
        # Expanded at load into one low-rank term (§3.1, "Other methods fit
        # as well"); see expand_product for the factors.
        A, B = expand_product(adapter)
        out["terms"].append({"c": float(adapter["c"]), "A": A, "d": None, "B": B, "e": None})
        out["owned"] = {"A", "B"}
        return out
    if meth == "stack":
        members = adapter["members"]
        out = unfolded_slots(members[0], W, shared)
        for mem in members[1:]:
            out = stack(out, unfolded_slots(mem, W, shared))
        return out
    raise ValueError("unknown method %r" % (meth,))


def expand_product(adapter):
    """Low-rank factors (A [d_in, R], B [R, d_out]) with A B equal to the
    update of LoHa or LoKr without c.
      LoHa: (A1 B1) ⊙ (A2 B2) = Σ_{k,l} (A1[:,k] ⊙ A2[:,l]) (B1[k] ⊙ B2[l]),
            so column (k, l) of A is A1[:,k] ⊙ A2[:,l] and row (k, l) of B is
            B1[k] ⊙ B2[l]; R = r1 · r2.
      LoKr: C ⊗ (A B) = (C ⊗ A)(I_q ⊗ B) (mixed products), R = q · r, or
            (I_p ⊗ A)(C ⊗ B), R = p · r; the smaller R is taken."""
    if adapter["method"] == "loha":
        A1, B1 = _f64(adapter["A"]), _f64(adapter["B"])
        A2, B2 = _f64(adapter["A2"]), _f64(adapter["B2"])
        A = (A1[:, :, None] * A2[:, None, :]).reshape(A1.shape[0], -1)
        B = (B1[:, None, :] * B2[None, :, :]).reshape(-1, B1.shape[1])
        return A, B
    if adapter["method"] == "lokr":
        C, A0, B0 = _f64(adapter["C"]), _f64(adapter["A"]), _f64(adapter["B"])
        p, q = C.shape
        if q <= p:
            return np.kron(C, A0), np.kron(np.eye(q), B0)
        return np.kron(np.eye(p), A0), np.kron(C, B0)
    raise ValueError("not a product method: %r" % (adapter["method"],))


def normal_form_eval(x, W, slots):
    """Evaluate eq. (1) literally, slot by slot, with identity defaults."""
    x = _f64(x)
    W = _f64(W)
    xr = x if slots["R"] is None else x @ slots["R"]
    y = xr @ W
    if slots["s"] is not None:
        y = y * slots["s"]
    if slots["b"] is not None:
        y = y + slots["b"]
    for t in slots["terms"]:
        v = x @ t["A"]
        if t["d"] is not None:
            v = v * t["d"]
        u = v @ t["B"]
        if t["e"] is not None:
            u = u * t["e"]
        y = y + t["c"] * u
    return y


def fold(slots):
    """Apply every fold the fold rule allows (§3.2, appendix "Proposition A1,
    the 'if' direction").  Only owned tensors change; shared factors and W
    never do.  Returns new slots and the list of folds made, each as
    "slot->target" (e.g. "c->A")."""
    owned = slots["owned"]
    new = {"R": slots["R"], "s": slots["s"], "b": slots["b"], "terms": [],
           "owned": set(owned)}
    made = []
    for t in slots["terms"]:
        c, A, d, B, e = t["c"], t["A"], t["d"], t["B"], t["e"]
        # e folds into an owned B:  (VB) ⊙ e = V (B diag e).
        if e is not None and "B" in owned:
            B = B * e[None, :]
            e = None
            made.append("e->B")
        # d folds into an owned A (x(A diag d)) or an owned B (diag(d) B).
        if d is not None and "A" in owned:
            A = A * d[None, :]
            d = None
            made.append("d->A")
        elif d is not None and "B" in owned:
            B = d[:, None] * B
            d = None
            made.append("d->B")
        # c folds into the first owned neighbour among A, d, B, e.
        if c != 1.0:
            if "A" in owned:
                A = c * A
                made.append("c->A")
            elif "d" in owned:
                d = c * (d if d is not None else np.ones(A.shape[1]))
                made.append("c->d")
            elif "B" in owned:
                B = c * B
                made.append("c->B")
            elif "e" in owned:
                e = c * (e if e is not None else np.ones(B.shape[1]))
                made.append("c->e")
            else:
                new["terms"].append({"c": c, "A": A, "d": d, "B": B, "e": e})
                continue
            c = 1.0
        new["terms"].append({"c": c, "A": A, "d": d, "B": B, "e": e})
    return new, made


def live_slots(slots):
    """Names of the non-identity slots that remain (s, b, R, d, e, c)."""
    live = []
    for k in ("R", "s", "b"):
        if slots[k] is not None:
            live.append(k)
    for t in slots["terms"]:
        for k in ("c", "d", "e"):
            v = t[k]
            if (k == "c" and v != 1.0) or (k != "c" and v is not None):
                if k not in live:
                    live.append(k)
    return live


# Table 1 of the page's §3.1: per method, whether it has a term and whether
# that term's factors are owned or shared, and which of the six slots hold a
# non-identity value before folding.  The ownership column is Table 1's; the
# non-identity slots follow from each method's definition (§2, §5.1).
_METHOD_SHAPE = {
    "lora": {"owned": ("A", "B"), "present": ("c",)},
    "dora": {"owned": ("A", "B"), "present": ("s", "c", "e")},
    "ia3": {"owned": (), "present": ("s",)},
    "ssf": {"owned": (), "present": ("s", "b")},
    "vera": {"owned": ("d", "e"), "present": ("c", "d", "e")},
    "oft": {"owned": ("R",), "present": ("R",)},
}


def fold_rule(owned, present):
    """Which present slots fold, and where, by the rule of the appendix
    "Folds": c folds when any of A, d, B, e is owned (into the first of
    them); d folds when A or B is owned; e folds when B is owned; s, b and R
    never fold.  Returns (folds, live) as sorted lists of strings."""
    owned = set(owned)
    folds, live = [], []
    for slot in present:
        if slot == "c":
            tgt = next((t for t in ("A", "d", "B", "e") if t in owned), None)
        elif slot == "d":
            tgt = next((t for t in ("A", "B") if t in owned), None)
        elif slot == "e":
            tgt = "B" if "B" in owned else None
        else:
            tgt = None
        if tgt is None:
            live.append(slot)
        else:
            folds.append("%s->%s" % (slot, tgt))
    return sorted(folds), sorted(live)


def member_table():
    """Table 1 derived by the fold rule: {method: {"owned", "folds", "live",
    "term"}} where term is "owned", "shared" or "none"."""
    table = {}
    for meth, shp in _METHOD_SHAPE.items():
        folds, live = fold_rule(shp["owned"], shp["present"])
        if meth in ("lora", "dora"):
            term = "owned"
        elif meth == "vera":
            term = "shared"
        else:
            term = "none"
        table[meth] = {"owned": sorted(shp["owned"]), "folds": folds,
                       "live": live, "term": term}
    return table


def stack(first, second):
    """Slots of F2(x; F1(x)): the member `second` applied to the output of
    `first` (appendix "Stacking").  Scale s1⊙s2, shift b1⊙s2 + b2, F1's
    terms scaled by s2 through their outer vector e, then F2's terms.  The
    second member must have R = I (its base path is F1's output)."""
    if second["R"] is not None:
        raise ValueError("the second member of a stack cannot have an input transform")

    def mul(u, v):
        if u is None:
            return None if v is None else v.copy()
        return u.copy() if v is None else u * v

    s2 = second["s"]
    out = {"R": first["R"], "s": mul(first["s"], s2), "terms": [],
           "owned": set(first["owned"]) | set(second["owned"])}
    b1 = first["b"]
    if b1 is None:
        out["b"] = None if second["b"] is None else second["b"].copy()
    else:
        b = b1 * s2 if s2 is not None else b1.copy()
        out["b"] = b if second["b"] is None else b + second["b"]
    for t in first["terms"]:
        nt = dict(t)
        nt["e"] = mul(t["e"], s2)
        out["terms"].append(nt)
    out["terms"].extend(dict(t) for t in second["terms"])
    return out
