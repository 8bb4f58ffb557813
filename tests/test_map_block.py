"""The order in which the MFMA kernels map workgroups to (head, tile)
(map_block, bwd_rope_apply_amd/csrc/tile.h), checked on the host over many
launch shapes by tests/map_block_check.cpp: a bijection, each XCD's fixed
head set, heaviest tiles first, and the head groups.  No GPU is needed."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_map_block_is_a_bijection_in_heaviest_first_order():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "map_block_check")
        r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            "-Wno-unused-command-line-argument",
                            f"-I{os.path.join(ROOT, 'include')}",
                            f"-I{os.path.join(ROOT, 'bwd_rope_apply_amd', 'csrc')}",
                            os.path.join(ROOT, "tests", "map_block_check.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(r.stdout, r.stderr[-2000:])
        assert r.returncode == 0, r.stdout + r.stderr[-2000:]
        assert " 0 failed" in r.stdout
