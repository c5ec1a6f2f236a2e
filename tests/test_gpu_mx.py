"""GPU parity with block scales: 8 E8M0 bytes per row, one per 32 elements."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (addr_to_host, assert_within_tolerance, device_tables, lib, oracle_sampled, sample_tokens,
                         small_device_tables, to_dev_ids)

pytestmark = pytest.mark.gpu
MX = "e8m0_block32"


def _say(msg):
    print(msg, flush=True)


def test_device_e8m0_fill_matches_host():
    _say("e8m0 fill, R=4096 and sampled full-size rows")
    t, c = device_tables(4096, 1001, MX)
    _, host_c = workloads.dense_tables(1001, 4096, MX)
    for s in range(48):
        assert np.array_equal(c[s].cpu().numpy(), host_c[s]), s
    R = 1 << 24
    t, c = device_tables(R, 1004, MX)
    rows = np.array([0, 7, 1 << 20, R - 1], dtype=np.int64)
    for s in (0, 29, 47):
        assert np.array_equal(c[s][torch.from_numpy(rows).cuda()].cpu().numpy(), workloads.e8m0_rows(1004, s, rows))


def test_mx_tiny_all_tokens():
    w = workloads.WORKLOADS[1]
    _say("e8m0 lookup, tiny workload, all tokens")
    ids, hist = workloads.make_ids(w)
    host_t, host_c = workloads.dense_tables(w.table_seed, w.rows, MX)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=MX)
    d_ids, d_hist = to_dev_ids(ids, hist)
    out = lib().gather_reduce(plan, lib().hash(plan, d_ids, d_hist))
    fused = lib().lookup(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    _, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, [w.rows] * 48, scale_format=MX)
    assert_within_tolerance(out.cpu().numpy(), want, abs_sum)
    assert torch.equal(fused, out)


def test_mx_block_scale_mapping_exact():
    """Code 1.0 everywhere, byte b of every row = 124 + b: element j of a module is 24 * 2^(j//32 - 3)."""
    _say("e8m0 block mapping, exact")
    R = 64
    host_t = [np.full((R, 256), 0x38, np.uint8) for _ in range(48)]
    host_c = [np.tile((124 + np.arange(8)).astype(np.uint8), (R, 1)) for _ in range(48)]
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=MX)
    ids = np.arange(100, dtype=np.int32).reshape(2, 50)
    out = lib().lookup(plan, *to_dev_ids(ids, None)).cpu().numpy()
    want = 24.0 * 2.0 ** (np.arange(256) // 32 - 3)
    assert np.array_equal(out, np.broadcast_to(want, out.shape).astype(np.float32))


def test_mx_special_exponents():
    """E8M0 0 (2^-127, subnormal in fp32) and 255 (NaN) through the kernel."""
    _say("e8m0 special exponents")
    R = 1
    host_t = [np.zeros((R, 256), np.uint8) for _ in range(48)]
    host_t[0][0] = 0x38  # 1.0 in module 0, sub-table 0
    host_t[24][0] = 0x38  # 1.0 in module 1, sub-table 24
    host_c = [np.full((R, 8), 127, np.uint8) for _ in range(48)]
    host_c[0][0] = [0, 1, 127, 254, 255, 126, 128, 100]
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=MX)
    out = lib().lookup(plan, *to_dev_ids(np.zeros((1, 3), np.int32), None))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    _, want, abs_sum = oracle.lookup(np.zeros((1, 3), np.int32), None, host_t, host_c, [1] * 48, scale_format=MX)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])  # single non-zero term per element: exact, including 2^-127
    assert np.all(got[:, 1] == 1.0)


@pytest.mark.parametrize("key", [3, 4])
def test_mx_workload_sampled(key):
    w = workloads.WORKLOADS[key]
    _say(f"e8m0 lookup, workload {key} sampled")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed, MX)
    plan = lib().Plan(t, c, scale_format=MX)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    out = lib().gather_reduce(plan, addr)
    fused = lib().lookup(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    tokens = sample_tokens(w.n_tok, 4096, 100 + key)
    want_addr, want, abs_sum = oracle_sampled(ids, hist, w.rows, w.table_seed, tokens, MX)
    assert np.array_equal(addr_to_host(addr), want_addr)
    assert_within_tolerance(out[torch.from_numpy(tokens).cuda()].cpu().numpy(), want, abs_sum)
    assert torch.equal(fused, out)


def test_mx_dedup_mode_equals_direct():
    _say("e8m0 dedup mode == direct")
    R = 2048
    host_t, host_c = workloads.dense_tables(66, R, MX)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=MX, vocab_size=5)
    ids = np.random.default_rng(3).integers(0, 5, size=(6, 400)).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    addr = lib().hash(plan, d_ids)
    direct = lib().gather_reduce(plan, addr)
    dd = lib().gather_reduce(plan, addr, out=torch.full_like(direct, float("nan")), groups=lib().dedup(plan, d_ids))
    torch.cuda.synchronize()
    assert torch.equal(dd, direct)
