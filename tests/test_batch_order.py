"""The batch order of the batched gather and the fused lookup, checked on the CPU: tests/batch_order_check.cpp is
compiled against the library's own header (batch_order.h) and enumerates the token of every wave of every block
for 1,450 batch shapes (1 to 80 sequences of 18 lengths, and a few large ones): every token is visited exactly once
and in bounds, blocks are 4 or 8 waves with 8 only where waves share gathers, and consecutive sequence groups of a
full tile are a multiple of 8 launch slots apart.  No GPU is used: block_token is host-callable."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_batch_order_visits_every_token_once(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "batch_order_check")
    r = subprocess.run([cc, "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "hashed_gram_memory_amd", "csrc"),
                        os.path.join(ROOT, "tests", "batch_order_check.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
