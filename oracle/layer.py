"""One adapted projection over a batch of many tenants, the canonical row
plan, and the parity metrics.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page: the Scute paper (arXiv 2611.01089).
  * §2 "The LoRA schedule": Punica's schedule sorts the batch so that the
    rows of each adapter are contiguous (a segment); each tile of rows
    belongs to one segment, so a tile reads one adapter's factors.
  * §4.1, route two: the shared-factor term runs as GEMMs over tiles of
    rows "whatever their adapters", skipping rows without such a term.
  * The faangrind "multi-lora-serving" page, "Batching requests that use
    different adapters": each row carries its slot index (slot_of_row).

Reading taken where the pages leave the plan open: rows are ordered by
(term class of their slot, slot, row index), with term class 0 = a term on
owned factors (one segment per slot), 1 = a term on shared factors (tiles
cross tenants), 2 = no term.  Rows whose slot is not loaded are computed as
the identity and raise a sticky flag.
"""
import numpy as np

from .methods import _f64, direct_forward, input_transform

TERM_OWNED, TERM_SHARED, TERM_NONE = 0, 1, 2


def layer_forward(x, W, slot_of_row, adapters, shared=None):
    """y[i] = F_{a(i)}(x[i]) by each method's direct definition, and the
    base output h[i] = (x[i] R_{a(i)}) W that the max-error bound scales.

    ``adapters`` maps slot -> adapter record; slots absent from it (and
    slot 0 unless given) are the identity.  Rows are grouped by slot only
    to call numpy once per tenant; every row is computed independently."""
    x = _f64(x)
    W = _f64(W)
    n = x.shape[0]
    d_in, d_out = W.shape
    y = np.zeros((n, d_out))
    h = np.zeros((n, d_out))
    slots = np.asarray(slot_of_row, dtype=np.int64)
    for sl in np.unique(slots):
        rows = np.nonzero(slots == sl)[0]
        ad = adapters.get(int(sl), {"method": "identity"})
        y[rows] = direct_forward(x[rows], W, ad, shared)
        R = input_transform(ad, d_in)
        h[rows] = (x[rows] @ R) @ W
    return y, h


def plan(slot_of_row, slot_class, tile_rows, has_R=None):
    """Canonical row plan.

    slot_class: sequence indexed by slot -> 0 owned term, 1 shared term,
    2 no term, or -1 for a slot that is not loaded.  Slot 0 is the identity
    (class 2).  A row whose slot is out of range or not loaded is remapped to
    slot 0 and sets ``invalid``.

    Returns a dict:
      perm       row ids in order of (class, slot, row)
      row_slot   effective slot per row (after remapping)
      seg_ptr, seg_slot  maximal runs of one slot in perm order
      class_ptr  [4]: start of each class in perm order, and n
      tiles      (p0, p1, kind, slot): class-0 segments cut into pieces of at
                 most tile_rows rows (kind 0, slot of the segment); the
                 class-1 and class-2 ranges cut into pieces of tile_rows
                 from their start (kind 1 / 2, slot -1)
      oft_tiles  (p0, p1, slot) for segments whose slot has R, cut likewise
      invalid    1 if any row was remapped
    """
    n = len(slot_of_row)
    ns = len(slot_class)
    row_slot = []
    invalid = 0
    for s in slot_of_row:
        s = int(s)
        if s < 0 or s >= ns or slot_class[s] < 0:
            row_slot.append(0)
            invalid = 1
        else:
            row_slot.append(s)
    cls = [int(slot_class[s]) if s != 0 else TERM_NONE for s in row_slot]
    perm = sorted(range(n), key=lambda i: (cls[i], row_slot[i], i))
    seg_ptr, seg_slot = [], []
    for p, i in enumerate(perm):
        if p == 0 or row_slot[i] != row_slot[perm[p - 1]]:
            seg_ptr.append(p)
            seg_slot.append(row_slot[i])
    seg_ptr.append(n)
    class_ptr = []
    for c in range(3):
        class_ptr.append(sum(1 for i in range(n) if cls[i] < c))
    class_ptr.append(n)
    tiles = []
    for j in range(len(seg_slot)):
        p0, p1 = seg_ptr[j], seg_ptr[j + 1]
        if cls[perm[p0]] != TERM_OWNED:
            continue
        for a in range(p0, p1, tile_rows):
            tiles.append((a, min(a + tile_rows, p1), TERM_OWNED, seg_slot[j]))
    for c in (TERM_SHARED, TERM_NONE):
        p0, p1 = class_ptr[c], class_ptr[c + 1]
        for a in range(p0, p1, tile_rows):
            tiles.append((a, min(a + tile_rows, p1), c, -1))
    oft_tiles = []
    if has_R is not None:
        for j in range(len(seg_slot)):
            if not has_R[seg_slot[j]]:
                continue
            p0, p1 = seg_ptr[j], seg_ptr[j + 1]
            for a in range(p0, p1, tile_rows):
                oft_tiles.append((a, min(a + tile_rows, p1), seg_slot[j]))
    return {"perm": perm, "row_slot": row_slot, "seg_ptr": seg_ptr,
            "seg_slot": seg_slot, "class_ptr": class_ptr, "tiles": tiles,
            "oft_tiles": oft_tiles, "invalid": invalid}


def parity_metrics(y, y_ref, h_ref, xw_ref):
    """Per-row error against the size of each row's adapter effect.

    err_i = ‖y_i − y_ref_i‖₂, eff_i = ‖y_ref_i − x_i W‖₂; ``mean_rel`` is the
    mean of err_i / eff_i over rows with eff_i > 0 and ``max_abs`` the
    largest elementwise |y − y_ref|, to be held under 2e-3 · max|h_ref|."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    err = np.sqrt(np.sum((y - y_ref) ** 2, axis=1))
    eff = np.sqrt(np.sum((y_ref - _f64(xw_ref)) ** 2, axis=1))
    mask = eff > 0
    rel = err[mask] / eff[mask]
    return {
        "mean_rel": float(rel.mean()) if rel.size else 0.0,
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "max_abs": float(np.max(np.abs(y - y_ref))) if y.size else 0.0,
        "max_h": float(np.max(np.abs(_f64(h_ref)))) if y.size else 0.0,
        "rows_with_effect": int(mask.sum()),
    }
