"""Checks on the gfx950 assembly of every HIP source (compiled here with hipcc; no GPU needed).

1. The direct global->LDS loads set M0 from inline asm, and the compiler ignores an asm clobber of
   M0 (a register it reserves). That is safe only while the compiler itself never uses M0 in the
   kernels that issue those loads: every M0 reference must be one of the helper's pairs,
   `s_mov_b32 m0, sN` immediately followed by the `global_load_lds_dword*` that reads it.
2. Packed fp32 VALU instructions (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32) are kept out of the
   library (the build disables the feature): none may appear.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_moe_transformer_02_amd import build as B

SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))
HAVE_HIPCC = bool(shutil.which(B.HIPCC)) or os.path.exists(B.HIPCC)


@pytest.fixture(scope="module", params=SOURCES)
def asm(request, tmp_path_factory):
    src = request.param
    out = tmp_path_factory.mktemp("isa") / (src + ".s")
    r = subprocess.run([B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ins = [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]
    return src, [ln for ln in ins if ln and not ln.startswith((".", "_")) and not ln.endswith(":")]


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not installed")
def test_m0_is_only_written_for_the_direct_lds_loads(asm):
    src, ins = asm
    for i, ln in enumerate(ins):
        if re.search(r"\bm0\b", ln):
            assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", ln), f"{src}: compiler use of m0: {ln!r}"
            assert ins[i + 1].startswith("global_load_lds_dword"), f"{src}: m0 write not followed by an LDS load"


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not installed")
def test_no_packed_fp32_instructions(asm):
    src, ins = asm
    bad = [ln for ln in ins if re.match(r"v_pk_(add|mul|fma)_f32\b", ln)]
    assert not bad, f"{src}: {bad[:3]}"
