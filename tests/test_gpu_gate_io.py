"""GPU parity of the gate inputs: un-reduced rows and caller-weighted sums."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import assert_within_tolerance, device_tables, lib, sample_tokens, small_device_tables, to_dev_ids

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("fmt", ["f32_row", "e8m0_block32"])
def test_rows_and_weighted_small(fmt):
    _say(f"gate inputs, small tables, {fmt}")
    R, N = 1024, 333
    host_t, host_c = workloads.dense_tables(21, R, fmt)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=fmt)
    rng = np.random.default_rng(5)
    addr = rng.integers(0, R, size=(N, 48)).astype(np.uint32)
    d_addr = torch.from_numpy(addr.view(np.int32)).cuda().view(torch.uint32)
    w = rng.uniform(-2, 2, size=(N, 48)).astype(np.float32)
    rows = lib().gather_rows(plan, d_addr)
    weighted = lib().gather_weighted(plan, d_addr, torch.from_numpy(w).cuda())
    ones = lib().gather_weighted(plan, d_addr, torch.ones((N, 48), device="cuda"))
    plain = lib().gather_reduce(plan, d_addr)
    torch.cuda.synchronize()
    want_rows = oracle.gather_rows(host_t, host_c, addr, fmt)
    assert_within_tolerance(rows.cpu().numpy(), want_rows, np.abs(want_rows))  # one rounding per element
    want, abs_sum = oracle.gather_weighted(host_t, host_c, addr, w, fmt)
    assert_within_tolerance(weighted.cpu().numpy(), want, abs_sum)
    assert torch.equal(ones, plain)


def test_weighted_full_size_sampled():
    w = workloads.WORKLOADS[4]
    _say("gate inputs, full-size tables, sampled tokens")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c)
    addr = lib().hash(plan, *to_dev_ids(ids, hist))
    rng = np.random.default_rng(12)
    weights = rng.uniform(0, 1, size=(w.n_tok, 48)).astype(np.float32)
    out = lib().gather_weighted(plan, addr, torch.from_numpy(weights).cuda())
    tokens = sample_tokens(w.n_tok, 2048, 77)
    sub_addr = addr.view(torch.int32)[torch.from_numpy(tokens).cuda()].contiguous().view(torch.uint32)
    sub_rows = lib().gather_rows(plan, sub_addr)
    torch.cuda.synchronize()
    a = oracle.hash_addresses(oracle.windows(ids, hist), oracle.multipliers(), [w.rows] * 48)[tokens]
    host = workloads.SparseHostTables(w.table_seed, w.rows)
    try:
        host.materialise(a)
        want, abs_sum = oracle.gather_weighted(host.tables, host.scales, a, weights[tokens])
        want_rows = oracle.gather_rows(host.tables, host.scales, a)
    finally:
        host.close()
    assert_within_tolerance(out[torch.from_numpy(tokens).cuda()].cpu().numpy(), want, abs_sum)
    assert_within_tolerance(sub_rows.cpu().numpy(), want_rows, np.abs(want_rows))
