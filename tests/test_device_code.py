"""CPU check of the device code as compiled for gfx950 (no GPU needed): every
kernel of the library has a body that ends in s_endpgm.  Undefined behaviour
in a kernel (a shift by the width of its operand, say) lets the compiler prove
the body unreachable and emit an entry point with no instructions, which a
wave would run past into whatever code follows; this catches that before any
launch."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["tiled.hip", "chunk.hip", "copy.hip"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="needs hipcc")
@pytest.mark.parametrize("src", SOURCES)
def test_every_kernel_has_a_body(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
           "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(ROOT, "bmmc_affine_index_amd", "csrc", "kernels", src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    s = out.read_text()
    kernels = re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", s, flags=re.M)
    assert kernels, "no kernels found in %s" % src
    for name in kernels:
        start = s.index("\n%s:" % name)
        end = s.index(".Lfunc_end", start)
        ins = [l.strip() for l in s[start:end].splitlines()[1:]]
        ins = [l for l in ins if l and not l.startswith((".", ";")) and not l.endswith(":")]
        assert ins and any(l.startswith("s_endpgm") for l in ins), name
