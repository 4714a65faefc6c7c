"""ctypes binding of libtpa.so with the names of include/tpa.h.

Argument marshalling only: device pointers and streams are plain integers
(``tensor.data_ptr()``, ``torch.cuda.current_stream().cuda_stream``); host
arrays are numpy float32.  Every call that returns a non-zero status raises
``TpaError`` with the library's message.  Importing this module fails loudly
if the library has not been built.
"""
import ctypes
import os
import re

import numpy as np

# torch ships its own HIP runtime under the same SONAME as ROCm's.  Loading it
# first makes libtpa.so bind to that single copy, so device pointers, streams
# and events created by torch are valid in the library.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tpa.h")

TPA_F32, TPA_F16, TPA_BF16 = 0, 1, 2
DTYPES = {"f32": TPA_F32, "f16": TPA_F16, "bf16": TPA_BF16}
METHODS = {"identity": 0, "lora": 1, "dora": 2, "ia3": 3, "vera": 4, "oft": 5, "ssf": 6, "stack": 7, "loha": 8, "lokr": 9}
(TPA_OPT_GEMM_SPLIT, TPA_OPT_SHRINK_SPLIT, TPA_OPT_TILE_ROWS, TPA_OPT_GEMM_PATH, TPA_OPT_SCALE_ROUTE,
 TPA_OPT_GEMM_NB, TPA_OPT_GEMM_GROUPS, TPA_OPT_GEMM_STAGES, TPA_OPT_OVERLAP, TPA_OPT_WIDE_TILE,
 TPA_OPT_FUSE_EXPAND, TPA_OPT_SHRINK_COLS) = (1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12)
LIVE_S, LIVE_B, LIVE_R, LIVE_D, LIVE_E = 1, 2, 4, 8, 16
FOLD_C_A, FOLD_E_B, FOLD_C_D, FOLD_D_A = 1, 2, 4, 8
STATUS = {0: "OK", -1: "INVALID", -2: "METHOD", -3: "NO_SLOT", -4: "UNKNOWN_SLOT",
          -5: "VALUE", -6: "WORKSPACE", -7: "HIP"}


class TpaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("tpa status %d (%s): %s" % (code, STATUS.get(code, "?"), msg))
        self.code = code


class tpa_adapter_desc(ctypes.Structure):
    _fields_ = ([("method", ctypes.c_int32), ("rank", ctypes.c_int32), ("oft_block", ctypes.c_int32),
                 ("c", ctypes.c_float)] + [(k, ctypes.c_void_p) for k in ("A", "B", "m", "l", "d", "e", "Q", "s", "b")]
                + [(k, ctypes.c_int32) for k in ("rank2", "kron_p", "kron_q", "reserved")]
                + [(k, ctypes.c_void_p) for k in ("A2", "B2", "C")])


class tpa_adapter_info(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("method", "live_mask", "fold_mask", "term_kind", "rank", "oft_block")]


class tpa_config(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("tile_rows", "gemm_path", "gemm_nb", "gemm_split", "gemm_kc",
                                              "shrink_split", "shrink_kc", "scale_route", "gemm_groups",
                                              "gemm_stages", "gemm_tile", "fused_expand", "shrink_cols",
                                              "shrink_in_gemm")]


class tpa_plan_host(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("perm", "row_slot", "seg_ptr", "seg_slot", "class_ptr", "tiles",
                                               "oft_tiles", "counts")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtpa.so is not built at %s; run __graft_entry__.build() or "
                          "python tenant_peft_adapter_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "tpa_method_info": [i32, P(tpa_adapter_info)],
        "tpa_layer_create": [i32, i32, i32, i32, vp, i32, i32, P(vp)],
        "tpa_layer_destroy": [vp],
        "tpa_vera_shared_set": [vp, i32, vp, vp, vp],
        "tpa_vera_shared_set_from": [vp, vp, vp, vp],
        "tpa_adapter_load": [vp, P(tpa_adapter_desc), P(i32), vp],
        "tpa_adapter_load_stack": [vp, P(tpa_adapter_desc), i32, P(i32), vp],
        "tpa_adapter_unload": [vp, i32, vp],
        "tpa_adapter_info_get": [vp, i32, P(tpa_adapter_info)],
        "tpa_workspace_size": [vp, i32, P(sz)],
        "tpa_layer_forward": [vp, vp, vp, i32, vp, vp, sz, vp],
        "tpa_layer_forward_noalloc": [vp, vp, vp, i32, vp, vp],
        "tpa_error_flag": [vp, P(i32), i32, vp],
        "tpa_plan_max_tiles": [vp, i32, P(i32), P(i32)],
        "tpa_plan_debug": [vp, vp, i32, vp, sz, P(tpa_plan_host), vp],
        "tpa_layer_set_option": [vp, i32, i32],
        "tpa_layer_config": [vp, i32, P(tpa_config)],
        "tpa_layer_plan_signature": [vp, P(ctypes.c_uint64)],
        "tpa_plan_accepts": [vp, vp, P(i32)],
        "tpa_plan_create": [P(vp)],
        "tpa_plan_destroy": [vp],
        "tpa_plan_size": [vp, i32, P(sz)],
        "tpa_plan_build": [vp, vp, vp, i32, vp, sz, vp],
        "tpa_layer_forward_planned": [vp, vp, vp, vp, vp, sz, vp],
        "tpa_group_workspace_size": [P(vp), i32, i32, P(sz)],
        "tpa_group_forward_planned": [P(vp), i32, vp, P(vp), P(vp), P(vp), P(sz), vp],
        "tpa_layer_set_stage_events": [vp, P(vp), i32],
        "tpa_timing_event_create": [P(vp)],
        "tpa_timing_event_destroy": [vp],
        "tpa_timing_event_elapsed": [vp, vp, P(ctypes.c_float)],
        "tpa_probe_copy": [vp, vp, sz, vp],
        "tpa_probe_read": [vp, sz, vp, vp],
        "tpa_probe_empty": [i32, vp],
        "tpa_probe_delay": [i32, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = i32
    lib.tpa_last_error.argtypes = []
    lib.tpa_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    return _lib


def header_symbols():
    """Function names declared in include/tpa.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:tpa_status|const char\*)\s+(tpa_\w+)\s*\(", text, re.M)))


def tpa_last_error():
    return _lib.tpa_last_error().decode()


def _check(code):
    if code != 0:
        raise TpaError(code, tpa_last_error())


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _info(i):
    return {k: getattr(i, k) for k, _ in tpa_adapter_info._fields_}


def tpa_method_info(method):
    out = tpa_adapter_info()
    _check(_lib.tpa_method_info(METHODS.get(method, method), ctypes.byref(out)))
    return _info(out)


def tpa_layer_create(device, d_in, d_out, dtype, W_ptr, max_slots, max_rank):
    h = ctypes.c_void_p()
    _check(_lib.tpa_layer_create(device, d_in, d_out, DTYPES.get(dtype, dtype), W_ptr, max_slots, max_rank,
                                 ctypes.byref(h)))
    return h.value


def tpa_layer_destroy(layer):
    _check(_lib.tpa_layer_destroy(layer))


def tpa_vera_shared_set(layer, r_v, A, B, stream=0):
    A, B = _f32(A), _f32(B)
    _check(_lib.tpa_vera_shared_set(layer, r_v, _ptr(A), _ptr(B), stream))


def tpa_vera_shared_set_from(layer, from_layer, B, stream=0):
    B = _f32(B)
    _check(_lib.tpa_vera_shared_set_from(layer, from_layer, _ptr(B), stream))


def _desc(method, rank=0, oft_block=0, c=1.0, A=None, B=None, m=None, l=None, d=None, e=None, Q=None, s=None,
          b=None, rank2=0, kron_p=0, kron_q=0, A2=None, B2=None, C=None):
    """A tpa_adapter_desc and the float32 arrays it points into (keep both
    alive until the call returns)."""
    keep = {k: _f32(v) for k, v in dict(A=A, B=B, m=m, l=l, d=d, e=e, Q=Q, s=s, b=b, A2=A2, B2=B2, C=C).items()}
    desc = tpa_adapter_desc(METHODS.get(method, method), rank, oft_block, c,
                            *[_ptr(keep[k]) for k in ("A", "B", "m", "l", "d", "e", "Q", "s", "b")],
                            rank2, kron_p, kron_q, 0, *[_ptr(keep[k]) for k in ("A2", "B2", "C")])
    return desc, keep


def tpa_adapter_load(layer, method, stream=0, **fields):
    """fields: the tpa_adapter_desc members the method uses (rank, c, A, ...)."""
    desc, keep = _desc(method, **fields)
    slot = ctypes.c_int32()
    _check(_lib.tpa_adapter_load(layer, ctypes.byref(desc), ctypes.byref(slot), stream))
    del keep
    return slot.value


def tpa_adapter_load_stack(layer, members, stream=0):
    """members: list of keyword dicts of tpa_adapter_load (method, rank, ...),
    applied in order."""
    made = [_desc(**mem) for mem in members]
    arr = (tpa_adapter_desc * len(made))(*[dsc for dsc, _ in made])
    slot = ctypes.c_int32()
    _check(_lib.tpa_adapter_load_stack(layer, arr, len(made), ctypes.byref(slot), stream))
    del made
    return slot.value


def tpa_adapter_unload(layer, slot, stream=0):
    _check(_lib.tpa_adapter_unload(layer, slot, stream))


def tpa_adapter_info_get(layer, slot):
    out = tpa_adapter_info()
    _check(_lib.tpa_adapter_info_get(layer, slot, ctypes.byref(out)))
    return _info(out)


def tpa_workspace_size(layer, n_max):
    out = ctypes.c_size_t()
    _check(_lib.tpa_workspace_size(layer, n_max, ctypes.byref(out)))
    return out.value


def tpa_layer_forward(layer, x_ptr, slot_of_row_ptr, n, out_ptr, ws_ptr, ws_bytes, stream=0):
    _check(_lib.tpa_layer_forward(layer, x_ptr, slot_of_row_ptr, n, out_ptr, ws_ptr, ws_bytes, stream))


NOALLOC_SCRATCH_BYTES = 64 << 20   # TPA_NOALLOC_SCRATCH_BYTES


def tpa_layer_forward_noalloc(layer, x_ptr, slot_of_row_ptr, n, out_ptr, stream=0):
    _check(_lib.tpa_layer_forward_noalloc(layer, x_ptr, slot_of_row_ptr, n, out_ptr, stream))


def tpa_layer_plan_signature(layer):
    out = ctypes.c_uint64()
    _check(_lib.tpa_layer_plan_signature(layer, ctypes.byref(out)))
    return out.value


def tpa_plan_accepts(plan, layer):
    out = ctypes.c_int32()
    _check(_lib.tpa_plan_accepts(plan, layer, ctypes.byref(out)))
    return bool(out.value)


def tpa_plan_create():
    h = ctypes.c_void_p()
    _check(_lib.tpa_plan_create(ctypes.byref(h)))
    return h.value


def tpa_plan_destroy(plan):
    _check(_lib.tpa_plan_destroy(plan))


def tpa_plan_size(layer, n_max):
    out = ctypes.c_size_t()
    _check(_lib.tpa_plan_size(layer, n_max, ctypes.byref(out)))
    return out.value


def tpa_plan_build(plan, layer, slot_of_row_ptr, n, plan_ptr, plan_bytes, stream=0):
    _check(_lib.tpa_plan_build(plan, layer, slot_of_row_ptr, n, plan_ptr, plan_bytes, stream))


def tpa_layer_forward_planned(layer, plan, x_ptr, out_ptr, ws_ptr, ws_bytes, stream=0):
    _check(_lib.tpa_layer_forward_planned(layer, plan, x_ptr, out_ptr, ws_ptr, ws_bytes, stream))


def tpa_group_workspace_size(layers, n_max):
    k = len(layers)
    arr = (ctypes.c_void_p * k)(*layers)
    out = (ctypes.c_size_t * k)()
    _check(_lib.tpa_group_workspace_size(arr, k, n_max, out))
    return list(out)


def tpa_group_forward_planned(layers, plan, x_ptrs, out_ptrs, ws_ptrs, ws_bytes, stream=0):
    k = len(layers)
    V = ctypes.c_void_p * k
    _check(_lib.tpa_group_forward_planned(V(*layers), k, plan, V(*x_ptrs), V(*out_ptrs), V(*ws_ptrs),
                                          (ctypes.c_size_t * k)(*ws_bytes), stream))


def tpa_error_flag(layer, clear=False, stream=0):
    out = ctypes.c_int32()
    _check(_lib.tpa_error_flag(layer, ctypes.byref(out), 1 if clear else 0, stream))
    return out.value


def tpa_plan_max_tiles(layer, n):
    mt, tr = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.tpa_plan_max_tiles(layer, n, ctypes.byref(mt), ctypes.byref(tr)))
    return mt.value, tr.value


def tpa_plan_debug(layer, slot_of_row_ptr, n, ws_ptr, ws_bytes, stream=0):
    mt, _ = tpa_plan_max_tiles(layer, n)
    arrs = {"perm": np.zeros(n, np.int32), "row_slot": np.zeros(n, np.int32), "seg_ptr": np.zeros(n + 1, np.int32),
            "seg_slot": np.zeros(max(n, 1), np.int32), "class_ptr": np.zeros(4, np.int32),
            "tiles": np.zeros(4 * max(mt, 1), np.int32), "oft_tiles": np.zeros(4 * max(mt, 1), np.int32),
            "counts": np.zeros(4, np.int32)}
    host = tpa_plan_host(*[arrs[k].ctypes.data for k, _ in tpa_plan_host._fields_])
    _check(_lib.tpa_plan_debug(layer, slot_of_row_ptr, n, ws_ptr, ws_bytes, ctypes.byref(host), stream))
    nseg, nt, no, inv = (int(v) for v in arrs["counts"])
    return {"perm": arrs["perm"].tolist(), "row_slot": arrs["row_slot"].tolist(),
            "seg_ptr": arrs["seg_ptr"][:nseg + 1].tolist(), "seg_slot": arrs["seg_slot"][:nseg].tolist(),
            "class_ptr": arrs["class_ptr"].tolist(),
            "tiles": [tuple(int(v) for v in arrs["tiles"][4 * i:4 * i + 4]) for i in range(nt)],
            "oft_tiles": [tuple(int(v) for v in arrs["oft_tiles"][4 * i:4 * i + 3]) for i in range(no)],
            "invalid": inv}


def tpa_layer_set_option(layer, key, value):
    _check(_lib.tpa_layer_set_option(layer, key, value))


def tpa_layer_config(layer, n):
    out = tpa_config()
    _check(_lib.tpa_layer_config(layer, n, ctypes.byref(out)))
    return {k: getattr(out, k) for k, _ in tpa_config._fields_}


def tpa_layer_set_stage_events(layer, events):
    """events: six hipEvent_t handles (ints), or None to stop recording."""
    if events is None:
        _check(_lib.tpa_layer_set_stage_events(layer, None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(_lib.tpa_layer_set_stage_events(layer, arr, len(events)))


def tpa_timing_event_create():
    h = ctypes.c_void_p()
    _check(_lib.tpa_timing_event_create(ctypes.byref(h)))
    return h.value


def tpa_timing_event_destroy(event):
    _check(_lib.tpa_timing_event_destroy(event))


def tpa_timing_event_elapsed(start, end):
    ms = ctypes.c_float()
    _check(_lib.tpa_timing_event_elapsed(start, end, ctypes.byref(ms)))
    return ms.value


def tpa_probe_copy(dst_ptr, src_ptr, nbytes, stream=0):
    _check(_lib.tpa_probe_copy(dst_ptr, src_ptr, nbytes, stream))


PROBE_READ_SINK_WORDS = 8192


def tpa_probe_read(src_ptr, nbytes, sink_ptr, stream=0):
    _check(_lib.tpa_probe_read(src_ptr, nbytes, sink_ptr, stream))


def tpa_probe_empty(count, stream=0):
    _check(_lib.tpa_probe_empty(count, stream))


def tpa_probe_delay(microseconds, stream=0):
    _check(_lib.tpa_probe_delay(microseconds, stream))
