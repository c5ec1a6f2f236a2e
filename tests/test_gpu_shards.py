"""Sub-table sharding (the multi-GPU layout that splits the 48 sub-tables), shown on one GPU.

Each of 8 shards owns 6 sub-tables; its plan points the other 42 at one zero
row, so its output is the partial per-module sum over its own sub-tables.
The partial sums, added in a fixed order (what a deterministic reduce-scatter
over the shards would do), must equal the full lookup within the fp32
tolerance of the reordered sum.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import assert_within_tolerance, lib, small_device_tables, to_dev_ids

pytestmark = pytest.mark.gpu


def test_eight_subtable_shards_sum_to_the_full_lookup():
    print("8 sub-table shards vs full lookup", flush=True)
    R = 4096
    host_t, host_c = workloads.dense_tables(314, R)
    t, c = small_device_tables(host_t, host_c)
    zero_t = torch.zeros((1, 256), dtype=torch.uint8, device="cuda")
    zero_c = torch.zeros(1, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(2)
    ids = rng.integers(0, 129280, size=(3, 700)).astype(np.int32)
    hist = rng.integers(0, 129280, size=(3, 3)).astype(np.int32)
    d_ids, d_hist = to_dev_ids(ids, hist)
    full = lib().lookup(lib().Plan(t, c), d_ids, d_hist)
    total = torch.zeros_like(full)
    for g in range(8):
        own = range(6 * g, 6 * g + 6)
        rows = [R if s in own else 1 for s in range(48)]
        tp = [t[s].data_ptr() if s in own else zero_t.data_ptr() for s in range(48)]
        cp = [c[s].data_ptr() if s in own else zero_c.data_ptr() for s in range(48)]
        shard = lib().Plan.from_pointers(rows, tp, cp, keep=(t, c, zero_t, zero_c))
        part = lib().lookup(shard, d_ids, d_hist)
        total += part  # fixed order: shard 0, 1, ..., 7
        # a shard's addresses for its own sub-tables are the full plan's (the hash depends only on ids and R)
    torch.cuda.synchronize()
    _, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, [R] * 48)
    assert_within_tolerance(total.cpu().numpy(), want, abs_sum)
    assert_within_tolerance(full.cpu().numpy(), want, abs_sum)
