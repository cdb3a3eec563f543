"""Resources of every kernel in the library, read from the AMD GPU assembly metadata of a
device-only compile (hipcc -S, gfx950; no GPU needed): no kernel uses private (scratch)
memory -- so a dispatch never makes the runtime allocate scratch, which the entry point for
callers that cannot allocate relies on -- none needs more than 256 VGPRs, and the LDS of each
fits the 160 KiB of a compute unit."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_lm_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def kernel_metadata(src: str, out_dir: str) -> list[dict]:
    from linear_cross_entropy_lm_amd.build import HIPCC_FLAGS
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    asm = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), src, "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    text = open(asm).read()
    meta = text[text.index("amdhsa.kernels:"):]
    kernels = []
    for block in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name or ".symbol:" not in block:
            continue
        get = lambda key: int(re.search(rf"\.{key}:\s+(\d+)", block).group(1))  # noqa: E731
        kernels.append({"name": name.group(1), "private": get("private_segment_fixed_size"),
                        "vgpr": get("vgpr_count"), "lds": get("group_segment_fixed_size")})
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
@pytest.mark.parametrize("src", ["flce.hip", "ce_logits.hip", "rmsnorm.hip"])
def test_no_kernel_uses_scratch(tmp_path, src):
    kernels = kernel_metadata(os.path.join(CSRC, src), str(tmp_path))
    assert len(kernels) >= 5
    for k in kernels:
        assert k["private"] == 0, f"{k['name']} uses {k['private']} bytes of private memory per lane"
        assert k["vgpr"] <= 256, k
        assert k["lds"] <= 160 * 1024, k
