"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-only logic (method metadata, argument validation
before any device call) behaves as documented."""
import ctypes
import json
import os

import pytest

from tenant_peft_adapter_amd import binding as B

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "table1_members.json")))["methods"]


def test_library_exports_every_header_symbol():
    names = B.header_symbols()
    assert len(names) >= 15
    lib = B.library()
    for n in names:
        assert hasattr(lib, n), n


def _decode(info):
    live = []
    for bit, name in ((B.LIVE_S, "s"), (B.LIVE_B, "b"), (B.LIVE_R, "R"), (B.LIVE_D, "d"), (B.LIVE_E, "e")):
        if info["live_mask"] & bit:
            live.append(name)
    folds = []
    for bit, name in ((B.FOLD_C_A, "c->A"), (B.FOLD_E_B, "e->B"), (B.FOLD_C_D, "c->d"), (B.FOLD_D_A, "d->A")):
        if info["fold_mask"] & bit:
            folds.append(name)
    return sorted(folds), sorted(live)


@pytest.mark.parametrize("meth", sorted(GOLD))
def test_method_info_is_table1(meth):
    info = B.tpa_method_info(meth)
    folds, live = _decode(info)
    assert folds == sorted(GOLD[meth]["folds"])
    assert live == sorted(GOLD[meth]["live"])
    want_term = {"lora": 1, "dora": 1, "vera": 2}.get(meth, 0)
    assert info["term_kind"] == want_term


def test_method_info_identity_and_unknown():
    info = B.tpa_method_info("identity")
    assert info["live_mask"] == 0 and info["fold_mask"] == 0 and info["term_kind"] == 0
    with pytest.raises(B.TpaError) as e:
        B.tpa_method_info(99)
    assert e.value.code == -2
    assert "unknown method" in B.tpa_last_error()


@pytest.mark.parametrize("args,code", [
    ((0, 100, 128, 1, 1, 8, 16), -1),      # d_in not a multiple of 64
    ((0, 128, 100, 1, 1, 8, 16), -1),      # d_out not a multiple of 128
    ((0, 128, 128, 7, 1, 8, 16), -1),      # unknown dtype
    ((0, 128, 128, 1, None, 8, 16), -1),   # null W
    ((0, 128, 128, 1, 1, 1, 16), -1),      # max_slots < 2
    ((0, 128, 128, 1, 1, 8, 0), -1),       # max_rank < 1
    ((0, 128, 128, 1, 1, 8, 513), -1),     # max_rank > 512
])
def test_layer_create_validates_before_touching_a_device(args, code):
    with pytest.raises(B.TpaError) as e:
        B.tpa_layer_create(*args)
    assert e.value.code == code


def test_null_layer_calls_fail_cleanly():
    lib = B.library()
    assert lib.tpa_layer_forward(None, None, None, 1, None, None, 0, None) == -1
    assert lib.tpa_adapter_unload(None, 1, None) == -1
    assert lib.tpa_layer_destroy(None) == 0
    out = ctypes.c_size_t()
    assert lib.tpa_workspace_size(None, 4, ctypes.byref(out)) == -1


C_CONSUMER = r"""
#include <stddef.h>
#include <stdio.h>
#include "tpa.h"
int main(void) {
  tpa_adapter_info info;
  if (tpa_method_info(TPA_LOHA, &info) != TPA_OK) return 2;
  printf("%zu %zu %zu %zu %zu %zu %zu %d %d\n", sizeof(tpa_adapter_desc), offsetof(tpa_adapter_desc, b),
         offsetof(tpa_adapter_desc, rank2), offsetof(tpa_adapter_desc, A2), offsetof(tpa_adapter_desc, C),
         sizeof(tpa_config), sizeof(tpa_adapter_info), info.fold_mask, info.term_kind);
  return tpa_method_info(42, &info) == TPA_ERR_METHOD ? 0 : 3;
}
"""


def test_plain_c_consumer_and_struct_layouts(tmp_path):
    """The header is plain C: a C99 program compiled with gcc includes it,
    links libtpa.so and calls a host-only entry point; the structs it sees
    have the layout the ctypes binding declares."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(B.HEADER), str(src), "-o", str(exe),
                    "-L", libdir, "-ltpa", "-Wl,-rpath," + libdir], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    size, off_b, off_rank2, off_a2, off_c, cfg, info, fold, term = map(int, res.stdout.split())
    assert size == ctypes.sizeof(B.tpa_adapter_desc)
    assert off_b == B.tpa_adapter_desc.b.offset
    assert off_rank2 == B.tpa_adapter_desc.rank2.offset
    assert off_a2 == B.tpa_adapter_desc.A2.offset
    assert off_c == B.tpa_adapter_desc.C.offset
    assert cfg == ctypes.sizeof(B.tpa_config)
    assert info == ctypes.sizeof(B.tpa_adapter_info)
    assert (fold, term) == (B.FOLD_C_A, 1)


def _fake_layer(d_in=64, d_out=128, dtype=None):
    """An AdaptedLayer shell over a CPU weight (no library handle): enough to
    exercise the wrapper's argument checks, which run before any C-ABI call."""
    import torch
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    L = object.__new__(AdaptedLayer)
    L.W = torch.zeros((d_out, d_in), dtype=dtype or torch.float16)
    L.d_out, L.d_in = d_out, d_in
    L.handle = None
    return L


def test_wrapper_accepts_well_formed_arguments():
    import torch
    L = _fake_layer()
    x = torch.zeros((5, 64), dtype=torch.float16)
    sor = torch.zeros(5, dtype=torch.int32)
    out = torch.zeros((5, 128), dtype=torch.float16)
    assert L.check_forward_args(x, sor, out) == 5
    assert L.check_forward_args(x[:0], sor[:0]) == 0


@pytest.mark.parametrize("case", ["x_narrow", "x_dtype", "x_strided", "x_1d", "sor_int64", "sor_short",
                                  "sor_strided", "out_shape", "out_dtype", "out_alias", "x_not_tensor"])
def test_wrapper_rejects_mismatched_tensors_before_any_launch(case):
    """A narrower or wider x, another dtype, a non-contiguous view, int64 slot
    ids or a wrong-size output would make the kernels read or write past the
    tensors (or pick wrong slots): the wrapper raises ValueError first.  The
    layer shell has no library handle, so reaching the C ABI would fail with
    another error."""
    import torch
    L = _fake_layer()
    x = torch.zeros((5, 64), dtype=torch.float16)
    sor = torch.zeros(5, dtype=torch.int32)
    out = torch.zeros((5, 128), dtype=torch.float16)
    if case == "x_narrow":
        x = torch.zeros((5, 32), dtype=torch.float16)
    elif case == "x_dtype":
        x = torch.zeros((5, 64), dtype=torch.float32)
    elif case == "x_strided":
        x = torch.zeros((5, 128), dtype=torch.float16)[:, ::2]
    elif case == "x_1d":
        x = torch.zeros(64, dtype=torch.float16)
    elif case == "sor_int64":
        sor = torch.zeros(5, dtype=torch.int64)
    elif case == "sor_short":
        sor = torch.zeros(4, dtype=torch.int32)
    elif case == "sor_strided":
        sor = torch.zeros(10, dtype=torch.int32)[::2]
    elif case == "out_shape":
        out = torch.zeros((5, 64), dtype=torch.float16)
    elif case == "out_dtype":
        out = torch.zeros((5, 128), dtype=torch.bfloat16)
    elif case == "out_alias":
        L = _fake_layer(d_in=128)
        x = torch.zeros((5, 128), dtype=torch.float16)
        out = x
    elif case == "x_not_tensor":
        x = [[0.0] * 64] * 5
    with pytest.raises(ValueError):
        L.forward(x, sor, out=out)


def _decl_comments():
    """(name, text) per function declared in include/tpa.h: the declaration
    with the comment lines directly above it."""
    import re
    lines = open(B.HEADER).read().split("\n")
    out = []
    for i, l in enumerate(lines):
        m = re.match(r"^(?:tpa_status|const char\*)\s+(tpa_\w+)\s*\(", l)
        if not m:
            continue
        block = []
        k = i
        while True:                                   # the declaration itself
            block.append(lines[k])
            if lines[k].rstrip().endswith(";") or "; /*" in lines[k]:
                break
            k += 1
        j = i - 1
        while j >= 0 and re.match(r"^\s*(/\*|\*|//)", lines[j]):   # its comment
            block.append(lines[j])
            j -= 1
        out.append((m.group(1), "\n".join(block)))
    return out


def test_every_header_declaration_cites_a_passage():
    import re
    decls = _decl_comments()
    assert len(decls) == len(B.header_symbols())
    # The no-allocation forward is not a step of the pages: its comment names
    # the callers it serves instead.
    missing = [n for n, t in decls if n != "tpa_layer_forward_noalloc" and
               not re.search(r"§|Table|[Aa]ppendix|eq\. \(|\"multi-lora-serving\" page", t)]
    assert not missing, missing
    noalloc = dict(decls)["tpa_layer_forward_noalloc"]
    assert "cannot allocate" in noalloc


def test_noalloc_scratch_size_matches_the_header():
    import re
    text = open(B.HEADER).read()
    m = re.search(r"#define TPA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
