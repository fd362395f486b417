"""Resource checks on the gfx950 code the build produces (CPU only: hipcc cross-compiles).

The attention kernel's performance depends on every value staying in registers:
a variant that spills VGPRs to scratch still computes the right result (the GPU
parity tests pass) but runs several times slower.  These checks read the kernel
descriptors hipcc emits for each source under csrc/ and fail on any scratch use
or on more LDS than a gfx950 workgroup can have.
"""
import os
import re
import shutil
import subprocess

import pytest

from packed_full_attention_amd import build as B

LDS_LIMIT = 160 * 1024  # bytes of LDS one gfx950 workgroup can allocate


def _kernels(src: str, tmp_path) -> dict:
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.DEVICE_FLAGS, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
           "-o", str(out), src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    kernels = {}
    # Metadata: one "- .args: ..." block per kernel, with .name and the counts.
    for block in re.split(r"\n  - \.", text.split("amdhsa.kernels:", 1)[1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = {}
        for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size",
                    "group_segment_fixed_size", "vgpr_count"):
            m = re.search(r"\." + key + r":\s+(\d+)", block)
            if m:
                fields[key] = int(m.group(1))
        kernels[name.group(1)] = fields
    return kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", [s for s in B.sources() if s.endswith(".hip")], ids=os.path.basename)
def test_no_scratch_and_lds_within_limit(src, tmp_path):
    kernels = _kernels(src, tmp_path)
    assert kernels, "no kernel descriptors found"
    for name, f in kernels.items():
        assert f.get("vgpr_spill_count", 0) == 0, (name, f)
        assert f.get("private_segment_fixed_size", 0) == 0, (name, f)
        assert f.get("group_segment_fixed_size", 0) <= LDS_LIMIT, (name, f)
