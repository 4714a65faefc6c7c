"""A thin object wrapper over the C ABI for one adapted projection.

PyTorch supplies device memory (weights, inputs, outputs, workspace) and
the stream; every step of the computation runs in libtpa.so's kernels.
"""
import numpy as np
import torch

from . import binding as B

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_TPA_OF_TORCH = {torch.float32: B.TPA_F32, torch.float16: B.TPA_F16, torch.bfloat16: B.TPA_BF16}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check_rows(name, t, n, width, dtype, device):
    """t must be a contiguous [n, width] tensor of `dtype` on `device`; the
    kernels read and write exactly that many elements from its data pointer."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, the layer's weight on %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, the layer computes in %s" % (name, t.dtype, dtype))
    if t.dim() != 2 or tuple(t.shape) != (n, width):
        raise ValueError("%s has shape %s, expected (%d, %d)" % (name, tuple(t.shape), n, width))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_slots(slot_of_row, n, device):
    """slot_of_row must be a contiguous int32 vector of n entries on `device`
    (an int64 vector would be read as twice as many int32 slots)."""
    if not isinstance(slot_of_row, torch.Tensor):
        raise ValueError("slot_of_row must be a torch tensor")
    if slot_of_row.device != device:
        raise ValueError("slot_of_row is on %s, the layer's weight on %s" % (slot_of_row.device, device))
    if slot_of_row.dtype != torch.int32:
        raise ValueError("slot_of_row has dtype %s, expected torch.int32" % slot_of_row.dtype)
    if slot_of_row.dim() != 1 or slot_of_row.numel() != n:
        raise ValueError("slot_of_row has shape %s, expected (%d,)" % (tuple(slot_of_row.shape), n))
    if not slot_of_row.is_contiguous():
        raise ValueError("slot_of_row must be contiguous")


def _check_ws(ws, device):
    """A caller's workspace must be a contiguous, 256-byte aligned tensor on
    the layer's device; its size is checked by the library, which refuses a
    short one (-6) before launching anything."""
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    if ws.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")


class AdaptedLayer:
    """One projection y = F_{slot_of_row[i]}(x[i]) over a shared weight W
    ([d_out, d_in], an nn.Linear weight on the GPU)."""

    def __init__(self, W, max_slots=64, max_rank=256):
        if not W.is_cuda or W.dim() != 2:
            raise ValueError("W must be a 2-D CUDA tensor [d_out, d_in]")
        self.W = W.contiguous()
        self.d_out, self.d_in = self.W.shape
        self.dtype = _TPA_OF_TORCH[self.W.dtype]
        self.device = self.W.device.index or 0
        self.handle = B.tpa_layer_create(self.device, self.d_in, self.d_out, self.dtype, self.W.data_ptr(),
                                         max_slots, max_rank)
        self._ws = None
        self._ws_n = 0     # rows the current workspace was checked for (0: check again)
        self._ws_max = 0   # most rows asked for so far

    def close(self):
        if self.handle:
            B.tpa_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_vera_shared(self, A, Bm):
        A = np.asarray(A, np.float32)
        B.tpa_vera_shared_set(self.handle, A.shape[1], A, Bm, _stream())

    def set_vera_shared_from(self, other, Bm):
        """VeRA's pair with other's stored A (read once by a group forward
        over projections of one input) and this layer's own B."""
        B.tpa_vera_shared_set_from(self.handle, other.handle, Bm, _stream())

    @staticmethod
    def _kwargs(rec):
        meth = rec["method"]
        kw = {}
        if meth in ("lora", "dora"):
            kw = dict(rank=rec["A"].shape[1], c=rec["c"], A=rec["A"], B=rec["B"], m=rec.get("m"))
        elif meth == "ia3":
            kw = dict(l=rec["l"])
        elif meth == "ssf":
            kw = dict(s=rec["s"], b=rec["b"])
        elif meth == "vera":
            kw = dict(c=rec.get("c", 1.0), d=rec["d"], e=rec["e"])
        elif meth == "oft":
            kw = dict(oft_block=rec["Q"].shape[1], Q=rec["Q"])
        elif meth == "loha":
            kw = dict(rank=rec["A"].shape[1], rank2=rec["A2"].shape[1], c=rec["c"], A=rec["A"], B=rec["B"],
                      A2=rec["A2"], B2=rec["B2"])
        elif meth == "lokr":
            kw = dict(rank=rec["A"].shape[1], kron_p=rec["C"].shape[0], kron_q=rec["C"].shape[1], c=rec["c"],
                      C=rec["C"], A=rec["A"], B=rec["B"])
        kw["method"] = meth
        return kw

    def load(self, rec):
        """Admit an adapter given as a raw-parameter record (method name and
        numpy arrays in the paper's math layout); returns its slot.  A record
        {"method": "stack", "members": [...]} admits the members as one
        stacked slot, applied in list order."""
        self._ws_n = 0
        if rec["method"] == "stack":
            return B.tpa_adapter_load_stack(self.handle, [self._kwargs(m) for m in rec["members"]], _stream())
        return B.tpa_adapter_load(self.handle, stream=_stream(), **self._kwargs(rec))

    def unload(self, slot):
        self._ws_n = 0
        B.tpa_adapter_unload(self.handle, slot, _stream())

    def info(self, slot):
        return B.tpa_adapter_info_get(self.handle, slot)

    def set_option(self, key, value):
        B.tpa_layer_set_option(self.handle, key, value)
        self._ws = None

    def config(self, n):
        return B.tpa_layer_config(self.handle, n)

    def workspace(self, n):
        """A workspace for up to n rows.  Its size also depends on the loaded
        slots, so loads and unloads make the next call check it again."""
        if self._ws is None or self._ws_n < n:
            size = B.tpa_workspace_size(self.handle, max(n, self._ws_max))
            if self._ws is None or self._ws.numel() < size:
                self._ws = torch.empty(max(size, 256), dtype=torch.uint8, device=self.W.device)
            self._ws_max = max(n, self._ws_max)
            self._ws_n = self._ws_max
        return self._ws

    def check_forward_args(self, x, slot_of_row=None, out=None, n=None):
        """Raise ValueError unless x ([n, d_in]), slot_of_row (int32 [n]) and
        out ([n, d_out]) are contiguous tensors of the layer's dtype (int32
        for the slots) on the weight's device, and out does not alias x."""
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x must be a 2-D tensor [n, d_in]")
        n = x.shape[0] if n is None else n
        _check_rows("x", x, n, self.d_in, self.W.dtype, self.W.device)
        if slot_of_row is not None:
            _check_slots(slot_of_row, n, self.W.device)
        if out is not None:
            _check_rows("out", out, n, self.d_out, self.W.dtype, self.W.device)
            if n > 0 and out.data_ptr() == x.data_ptr():
                raise ValueError("out may not alias x")
        return n

    def forward(self, x, slot_of_row, out=None, ws=None):
        n = self.check_forward_args(x, slot_of_row, out)
        if out is None:
            out = torch.empty((n, self.d_out), dtype=self.W.dtype, device=self.W.device)
        if n == 0:
            return out
        if ws is None:
            ws = self.workspace(n)
        else:
            _check_ws(ws, self.W.device)
        B.tpa_layer_forward(self.handle, x.data_ptr(), slot_of_row.data_ptr(), n, out.data_ptr(), ws.data_ptr(),
                            ws.numel() * ws.element_size(), _stream())
        return out

    def plan_signature(self):
        """Layers with equal signatures can share a RowPlan."""
        return B.tpa_layer_plan_signature(self.handle)

    def forward_planned(self, plan, x, out=None, ws=None):
        """Forward of the rows of a RowPlan built by a layer with the same
        slot classes (the plan kernel is not run again)."""
        n = plan.n
        self.check_forward_args(x, None, out, n=n)
        if out is None:
            out = torch.empty((n, self.d_out), dtype=self.W.dtype, device=self.W.device)
        if n == 0:
            return out
        if ws is None:
            ws = self.workspace(n)
        else:
            _check_ws(ws, self.W.device)
        B.tpa_layer_forward_planned(self.handle, plan.handle, x.data_ptr(), out.data_ptr(), ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream())
        return out

    def plan(self, slot_of_row):
        n = slot_of_row.numel()
        _check_slots(slot_of_row, n, self.W.device)
        ws = self.workspace(max(n, 1))
        return B.tpa_plan_debug(self.handle, slot_of_row.data_ptr(), n, ws.data_ptr(), ws.numel(), _stream())

    def error_flag(self, clear=False):
        return B.tpa_error_flag(self.handle, clear, _stream())


class RowPlan:
    """A row plan built once by one layer and reused by every layer with the
    same slot classes (tpa_plan_build / tpa_layer_forward_planned)."""

    def __init__(self, layer, n_max):
        self.handle = B.tpa_plan_create()
        size = B.tpa_plan_size(layer.handle, n_max)
        self.buf = torch.empty(max(size, 256), dtype=torch.uint8, device=layer.W.device)
        self.n = 0
        self.n_max = n_max

    def accepts(self, layer):
        """Whether layer may forward this plan's rows (tpa_plan_accepts)."""
        return B.tpa_plan_accepts(self.handle, layer.handle)

    def build(self, layer, slot_of_row):
        n = slot_of_row.numel() if isinstance(slot_of_row, torch.Tensor) else -1
        _check_slots(slot_of_row, n, layer.W.device)
        if n > self.n_max:
            raise ValueError("plan buffer sized for %d rows, got %d" % (self.n_max, n))
        self.n = n
        B.tpa_plan_build(self.handle, layer.handle, slot_of_row.data_ptr(), self.n, self.buf.data_ptr(),
                         self.buf.numel(), _stream())
        return self

    def close(self):
        if self.handle:
            B.tpa_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LayerGroup:
    """Projections of one fused layer (q, k, v or gate, up) that share a row
    plan, forwarded with one launch per kernel (tpa_group_forward_planned)."""

    def __init__(self, layers, n_max, ws=None):
        """ws: optional per-projection workspaces to use instead of fresh
        ones (groups that never run at the same time may share them)."""
        self.layers = list(layers)
        sizes = B.tpa_group_workspace_size([L.handle for L in self.layers], n_max)
        if ws is not None:
            if len(ws) != len(self.layers) or any(w.numel() < sz for w, sz in zip(ws, sizes)):
                raise ValueError("shared workspaces too small for this group")
            self.ws = list(ws)
        else:
            self.ws = [torch.empty(max(sz, 256), dtype=torch.uint8, device=L.W.device)
                       for L, sz in zip(self.layers, sizes)]

    def forward(self, plan, xs, outs=None):
        if len(xs) != len(self.layers) or (outs is not None and len(outs) != len(self.layers)):
            raise ValueError("one input (and output) per projection of the group")
        for i, L in enumerate(self.layers):
            L.check_forward_args(xs[i], None, None if outs is None else outs[i], n=plan.n)
        if outs is None:
            outs = [torch.empty((plan.n, L.d_out), dtype=L.W.dtype, device=L.W.device) for L in self.layers]
        B.tpa_group_forward_planned([L.handle for L in self.layers], plan.handle, [x.data_ptr() for x in xs],
                                    [o.data_ptr() for o in outs], [w.data_ptr() for w in self.ws],
                                    [w.numel() for w in self.ws], _stream())
        return outs
