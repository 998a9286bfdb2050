"""Properties of the generated gfx950 code, checked on the host (no GPU): each
kernel source is compiled to device assembly with the library's own flags.

* M0 is written only by the direct global->LDS copy helper, right before its
  load: the compiler reserves M0 and cannot be told that an asm statement
  overwrites it, so any use of its own would be silently corrupted.
* No kernel spills to scratch (private segment size 0).
* No packed-fp32 VALU instructions (the build disables them).
"""
import os
import re
import subprocess

import pytest

from triangular_pair_attention_amd import build as B

def _has_kernels(src):
    with open(os.path.join(B.CSRC, src)) as f:
        return "__global__" in f.read()


KERNELS = tuple(u for u in B.units() if u[0].endswith(".hip") and _has_kernels(u[0]))


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module", params=KERNELS, ids=lambda u: u[1])
def asm(request, tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    src, name, extra = request.param
    out = tmp_path_factory.mktemp("asm") / (name + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    cmd = [cc, *flags, *extra, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    return name, out.read_text().splitlines()


def _instructions(lines):
    for ln in lines:
        s = ln.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            yield s


def test_m0_only_set_by_the_lds_copy(asm):
    name, lines = asm
    ins = list(_instructions(lines))
    for n, s in enumerate(ins):
        if re.search(r"\bm0\b", s):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", s), f"{name}: compiler use of m0: {s}"
            assert ins[n + 1] == "s_nop 0" and ins[n + 2].startswith("global_load_lds_dwordx4"), \
                f"{name}: m0 write not followed by the LDS copy"


def test_no_scratch_spills(asm):
    name, lines = asm
    sizes = [int(l.split()[-1]) for l in lines if ".amdhsa_private_segment_fixed_size" in l]
    assert sizes, f"{name}: no kernel descriptors found"
    assert all(s == 0 for s in sizes), f"{name}: private segment sizes {sizes}"


def test_no_packed_fp32(asm):
    name, lines = asm
    bad = [s for s in _instructions(lines) if re.match(r"v_pk_(fma|mul|add)_f32\b", s)]
    assert not bad, f"{name}: {bad[:3]}"
