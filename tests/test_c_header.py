"""The header is a plain C interface: a C99 program that includes
include/h3attn.h compiles with gcc, links against libh3attn.so and calls the
entry points that need no GPU (version, status strings, a call that argument
validation rejects, a size query).  CPU only."""
import os
import shutil
import subprocess

import pytest

from packed_full_attention_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

PROGRAM = r"""
#include "h3attn.h"
#include <stdio.h>
#include <string.h>
int main(void) {
  if (h3attn_abi_version() != H3ATTN_ABI_VERSION) return 1;
  if (strcmp(h3attn_strerror(H3A_OK), "success") != 0) return 2;
  if (h3attn_forward(NULL, NULL, NULL, NULL, 16, 1, 0.125f, (hipStream_t)0) != H3A_EINVAL) return 3;
  if (strstr(h3attn_last_error(), "null") == NULL) return 4;
  if (h3attn_vt_bytes(65, 1) != 128 * 128 * 2) return 5;
  if (h3attn_rope_table_bytes(10, 2) != 10 * 96 * 4) return 6;
  puts("ok");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE), reason="needs gcc and ROCm headers")
def test_c99_program_compiles_links_and_runs(tmp_path):
    b.load_library()  # the built library must exist
    src = tmp_path / "use_h3attn.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_h3attn"
    libdir = os.path.dirname(b.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
           ROCM_INCLUDE, str(src), "-L", libdir, "-l:libh3attn.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout, run.stderr)
