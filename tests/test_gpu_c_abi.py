"""The C ABI from a plain C program (no Python, no torch in its process), checked against the oracle: hash,
gather, fused lookup, the batch-order gather, and dedup with both dedup-mode calls."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from gpu_support import assert_within_tolerance

pytestmark = pytest.mark.gpu
DEMO = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "hashed_gram_memory_amd", "c_abi_demo")


def test_c_program_matches_oracle(tmp_path):
    n_tok, rows, seed = 777, 4096, 1001
    out_file = tmp_path / "demo.bin"
    print(f"c_abi_demo {n_tok} tokens", flush=True)
    r = subprocess.run([DEMO, str(out_file), str(n_tok), str(rows), str(seed)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(out_file, dtype=np.uint8)
    o = 0
    ids = raw[o:o + 4 * n_tok].view(np.int32)
    o += 4 * n_tok
    addr = raw[o:o + 4 * 48 * n_tok].view(np.uint32).reshape(n_tok, 48)
    o += 4 * 48 * n_tok
    out = raw[o:o + 4 * 512 * n_tok].view(np.float32).reshape(n_tok, 2, 256)
    o += 4 * 512 * n_tok
    fused = raw[o:o + 4 * 512 * n_tok].view(np.float32).reshape(n_tok, 2, 256)
    assert np.array_equal(ids, (np.arange(n_tok) * 7) % 129280)
    host_t, host_c = workloads.dense_tables(seed, rows)
    want_addr, want, abs_sum = oracle.lookup(ids.reshape(1, n_tok), None, host_t, host_c, [rows] * 48)
    assert np.array_equal(addr, want_addr)
    assert_within_tolerance(out, want, abs_sum)
    assert np.array_equal(fused, out)
    # the program's dedup case (ids i mod 5; dedup-mode results compared bitwise with the direct lookup inside it)
    groups = [int(line.split(":")[1]) for line in r.stdout.splitlines() if line.startswith("dedup groups:")]
    rep = (np.arange(n_tok) % 5).astype(np.int32).reshape(1, n_tok)
    assert groups == [oracle.dedup(oracle.windows(rep))[2]]
