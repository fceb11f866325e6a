"""The packed tile layouts of the statistics pass and the attention kernel, checked on
the host against the MFMA operand and accumulator definitions (tile_layout_check.hip)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_attention_43_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_tile_layouts(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "tile_layout_check")
    subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
                    os.path.join(HERE, "tile_layout_check.hip"), "-o", exe],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout
