"""The direct global->LDS loads set M0 from inline asm, and the compiler ignores an asm clobber of
M0 (a register it reserves). This is safe only while the compiler itself never uses M0 in the
kernels that issue those loads. Compile them to gfx950 assembly (hipcc, no GPU needed) and check
that every M0 reference is one of the helper's pairs: `s_mov_b32 m0, sN` immediately followed by
the `global_load_lds_dword*` that reads it.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_moe_transformer_02_amd import build as B

SOURCES = [f for f in sorted(os.listdir(B.CSRC))
           if f.endswith(".hip") and re.search(r"\bdma(16|4)\(", open(os.path.join(B.CSRC, f)).read())]


@pytest.mark.skipif(not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES)
def test_m0_is_only_written_for_the_direct_lds_loads(src, tmp_path):
    out = tmp_path / (src + ".s")
    r = subprocess.run([B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ins = [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]
    ins = [ln for ln in ins if ln and not ln.startswith((".", "_")) and not ln.endswith(":")]
    pairs = 0
    for i, ln in enumerate(ins):
        if not re.search(r"\bm0\b", ln):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{src}: compiler use of m0: {ln!r}"
        assert ins[i + 1].startswith("global_load_lds_dword"), f"{src}: m0 write not followed by an LDS load: {ln!r}"
        pairs += 1
    assert pairs > 0
