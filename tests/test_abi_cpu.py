"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/tri_attn.h declares, and rejects bad arguments before
touching the HIP runtime."""
import ctypes
import math
import os
import subprocess

import pytest

from triangular_pair_attention_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def test_header_declares_the_abi():
    names = B.declared_functions()
    for n in ("tri_attn_create", "tri_attn_workspace_size", "tri_attn_forward", "tri_attn_destroy",
              "tri_attn_strerror", "tri_attn_get_workspace_layout", "tri_attn_project", "tri_attn_attend",
              "tri_attn_output", "tri_attn_forward_train"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for n in B.declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(B.declared_functions()) <= exported


def test_struct_layouts_match_header(tmp_path):
    """Sizes and field offsets of the binding's structs equal what a C
    compiler makes of include/tri_attn.h."""
    import shutil

    structs = (("tri_attn_config", B.tri_attn_config), ("tri_attn_weights", B.tri_attn_weights),
               ("tri_attn_workspace_layout", B.tri_attn_workspace_layout), ("tri_attn_grads", B.tri_attn_grads))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tri_attn.h"', "int main(void) {"]
    for cname, cls in structs:
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    include = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-I", include, str(src), "-o", str(exe)], check=True, capture_output=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for cname, cls in structs:
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(cls, fname).offset, f"{cname}.{fname}"


def test_strerror():
    assert B.tri_attn_strerror(0) == "ok"
    assert "invalid" in B.tri_attn_strerror(B.TRI_ATTN_ERR_INVALID_ARG)
    assert "workspace" in B.tri_attn_strerror(B.TRI_ATTN_ERR_WORKSPACE)
    assert "unknown" in B.tri_attn_strerror(12345)


def _create_rc(**kw):
    base = dict(pair_dim=128, num_heads=4, dtype=B.TRI_ATTN_BF16, ln_eps=1e-5, mask_fill=-1e9)
    base.update(kw)
    cfg = B.tri_attn_config(**base)
    w = B.tri_attn_weights(**{k: 16 for k in B.WEIGHT_FIELDS})  # never dereferenced: rejected first
    h = ctypes.c_void_p()
    return B.raw_call("tri_attn_create", ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)), h


@pytest.mark.parametrize("kw,code", [
    (dict(pair_dim=130, num_heads=4), B.TRI_ATTN_ERR_INVALID_ARG),   # D % h != 0
    (dict(num_heads=0), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(pair_dim=-4), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(dtype=7), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(ln_eps=0.0), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(ln_eps=math.nan), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(mask_fill=-1.0), B.TRI_ATTN_ERR_INVALID_ARG),              # not a masking value
    (dict(mask_fill=math.nan), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(ending_node=2), B.TRI_ATTN_ERR_INVALID_ARG),               # 0 or 1 only
    (dict(ending_node=-1), B.TRI_ATTN_ERR_INVALID_ARG),
    (dict(pair_dim=96, num_heads=3), B.TRI_ATTN_ERR_UNSUPPORTED),     # d = 32 but D = 96
    (dict(pair_dim=128, num_heads=2), B.TRI_ATTN_ERR_UNSUPPORTED),    # d = 64
    (dict(pair_dim=256, num_heads=8), B.TRI_ATTN_ERR_UNSUPPORTED),    # D = 256
])
def test_create_rejects_bad_config(kw, code):
    rc, h = _create_rc(**kw)
    assert rc == code
    assert h.value is None


def test_create_null_arguments():
    h = ctypes.c_void_p()
    assert B.raw_call("tri_attn_create", None, None, None, ctypes.byref(h)) == B.TRI_ATTN_ERR_INVALID_ARG
    cfg = B.tri_attn_config(128, 4, B.TRI_ATTN_F32, 1e-5, -1e9)
    assert B.raw_call("tri_attn_create", ctypes.byref(cfg), None, None, ctypes.byref(h)) == B.TRI_ATTN_ERR_INVALID_ARG
    w = B.tri_attn_weights(**{k: 16 for k in B.WEIGHT_FIELDS})
    w.b_out = None
    assert B.raw_call("tri_attn_create", ctypes.byref(cfg), ctypes.byref(w), None,
                      ctypes.byref(h)) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_create", ctypes.byref(cfg), ctypes.byref(w), None, None) == B.TRI_ATTN_ERR_INVALID_ARG


def test_null_handle_paths():
    n = ctypes.c_size_t()
    assert B.raw_call("tri_attn_workspace_size", None, 1, 8, ctypes.byref(n)) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_forward", None, 1, 1, 1, 1, 8, 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_project", None, 1, 1, 1, 8, 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_attend", None, 1, 8, 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_output", None, 1, 1, 8, 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_forward_train", None, 1, 1, 1, None, 1, 8, ctypes.c_double(0.1), ctypes.c_uint64(1),
                      ctypes.c_uint32(0), 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    g = B.tri_attn_grads()
    assert B.raw_call("tri_attn_backward_workspace_size", None, 1, 8, ctypes.byref(n)) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_backward_train", None, 1, 1, 1, 1, 8, ctypes.c_double(0.1), ctypes.c_uint64(1),
                      ctypes.c_uint32(0), ctypes.byref(g), 1, 1 << 20, None) == B.TRI_ATTN_ERR_INVALID_ARG
    lay = B.tri_attn_workspace_layout()
    assert B.raw_call("tri_attn_get_workspace_layout", None, 1, 8, ctypes.byref(lay)) == B.TRI_ATTN_ERR_INVALID_ARG
    assert B.raw_call("tri_attn_destroy", None) == B.TRI_ATTN_OK


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library(str(tmp_path / "nope.so"))
