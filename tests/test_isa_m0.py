"""The LDS-writing loads of spec_verify_linear's k_dma and of
spec_verify_linear_packed's k_packed are issued from inline assembly that sets
M0 (the LDS base of the load) itself.  That is sound only while the compiler
keeps no value of its own in M0 in those kernels: this test compiles each
source to gfx950 assembly and checks, for every instantiation, that each M0
access is one of those writes and that there is exactly one write per load.
Runs on the CPU (hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_accept_amd import _build

pytestmark = pytest.mark.timeout(300)


@pytest.mark.parametrize("source,kernel", [("spec_verify_linear.hip", "k_dma"),
                                           ("spec_verify_linear_packed.hip", "k_packed")])
def test_m0_only_set_by_the_lds_loads(tmp_path, source, kernel):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(_build.CSRC, source)
    out = tmp_path / "linear.s"
    cmd = [cc, *_build.COMMON, *_build.PER_FILE.get(source, []), "-x", "hip",
           "--cuda-device-only", "-S", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = {}
    name = None
    for line in out.read_text().splitlines():
        m = re.match(r"^(_Z\S*" + kernel + r"I\S*):", line)
        if m:
            name = m.group(1)
            kernels[name] = {"m0": 0, "set": 0, "loads": 0}
            continue
        if name is None:
            continue
        if line.strip() == "s_endpgm":
            name = None
            continue
        body = line.split(";")[0]
        if re.search(r"\bm0\b", body):
            kernels[name]["m0"] += 1
            if re.match(r"\s*s_mov_b32 m0, s\d+\s*$", body):
                kernels[name]["set"] += 1
        if "global_load_lds_dwordx4" in body:
            kernels[name]["loads"] += 1
    assert kernels, f"no {kernel} kernel in the assembly"
    for k, c in kernels.items():
        assert c["loads"] > 0, k
        assert c["m0"] == c["set"] == c["loads"], (k, c)
