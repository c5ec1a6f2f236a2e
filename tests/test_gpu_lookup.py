"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Hash addresses must match bit for bit; memory vectors must satisfy
|gpu - oracle| <= 1e-5 * sum|terms| per element (exact where every term is
zero, NaN where the oracle is NaN).  The fp32 sum of 24 terms in a fixed
order carries at most ~23 * 2^-24 * sum|terms| ~ 1.4e-6 * sum|terms| of
rounding error, so the bound holds with margin for any summation order.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (addr_to_host, assert_within_tolerance, device_tables, dummy_plan, lib,
                         mark_buffer_dirty, oracle_sampled, sample_tokens, small_device_tables, to_dev_ids)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------- generator

def test_device_fill_matches_host_generator_small():
    _say("fill small R=4096 seed 1001")
    t, c = device_tables(4096, 1001)
    host_t, host_c = workloads.dense_tables(1001, 4096)
    for s in range(48):
        assert np.array_equal(t[s].cpu().numpy(), host_t[s]), s
        assert np.array_equal(c[s].cpu().numpy(), host_c[s]), s


def test_device_fill_matches_host_generator_full_size_sampled():
    _say("fill full R=2^24 seed 1004 sampled rows")
    R = 1 << 24
    t, c = device_tables(R, 1004)
    rows = np.array([0, 1, 255, 4096, 1 << 20, (1 << 23) + 7, R - 2, R - 1], dtype=np.int64)
    idx = torch.from_numpy(rows).cuda()
    for s in (0, 1, 23, 24, 46, 47):
        hc, hs = workloads.table_rows(1004, s, rows)
        assert np.array_equal(t[s][idx].cpu().numpy(), hc), s
        assert np.array_equal(c[s][idx].cpu().numpy(), hs), s


# --------------------------------------------------------------------------- hash

@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_hash_bit_exact_workloads(key):
    w = workloads.WORKLOADS[key]
    _say(f"hash workload {key} ({w.name}) n_tok={w.n_tok}")
    ids, hist = workloads.make_ids(w)
    plan = dummy_plan(w.rows)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    want = oracle.hash_addresses(oracle.windows(ids, hist), oracle.multipliers(), [w.rows] * 48)
    assert np.array_equal(addr_to_host(addr), want)


@pytest.mark.parametrize("n_seq,seq_len,with_hist,rows", [
    (1, 1, False, 3), (1, 1, True, 1), (3, 5, True, 1000003), (7, 300, True, 1 << 32),
    (2, 1000, False, (1 << 32) - 1), (5, 257, False, 61), (64, 1, True, 1 << 20), (1, 4099, False, 2),
])
def test_hash_bit_exact_shapes(n_seq, seq_len, with_hist, rows):
    _say(f"hash shape {n_seq}x{seq_len} hist={with_hist} R={rows}")
    rng = np.random.default_rng(n_seq * 1000 + seq_len)
    ids = rng.integers(0, 1 << 31, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    hist = rng.integers(0, 1 << 31, size=(n_seq, 3), dtype=np.int64).astype(np.int32) if with_hist else None
    plan = dummy_plan(rows)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    want = oracle.hash_addresses(oracle.windows(ids, hist), oracle.multipliers(), [rows] * 48)
    assert np.array_equal(addr_to_host(addr), want)


def test_hash_custom_seed_and_mixed_rows():
    _say("hash custom seed, per-sub-table rows")
    rng = np.random.default_rng(9)
    rows = [int(r) for r in rng.integers(1, 1 << 32, size=48)]
    rows[0], rows[1], rows[47] = 1, 1 << 32, 4096
    t = torch.zeros((1, 256), dtype=torch.uint8, device="cuda")
    c = torch.zeros(1, dtype=torch.float32, device="cuda")
    plan = lib().Plan.from_pointers(rows, [t.data_ptr()] * 48, [c.data_ptr()] * 48, hash_seed=12345, keep=(t, c))
    assert plan.multipliers() == [int(v) for v in oracle.multipliers(12345).ravel()]
    ids = rng.integers(0, 129280, size=(4, 777)).astype(np.int32)
    addr = lib().hash(plan, *to_dev_ids(ids, None))
    torch.cuda.synchronize()
    want = oracle.hash_addresses(oracle.windows(ids), oracle.multipliers(12345), rows)
    assert np.array_equal(addr_to_host(addr), want)


# --------------------------------------------------------------------------- gather-reduce

def test_lookup_tiny_all_tokens():
    w = workloads.WORKLOADS[1]
    _say("lookup workload 1 (tiny) all tokens")
    ids, hist = workloads.make_ids(w)
    host_t, host_c = workloads.dense_tables(w.table_seed, w.rows)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    addr = lib().hash(plan, *to_dev_ids(ids, hist))
    out = lib().gather_reduce(plan, addr)
    torch.cuda.synchronize()
    want_addr, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, [w.rows] * 48)
    assert np.array_equal(addr_to_host(addr), want_addr)
    assert_within_tolerance(out.cpu().numpy(), want, abs_sum)


@pytest.mark.parametrize("n_tok", [1, 2, 3, 4, 5, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1000, 4099])
def test_gather_ragged_token_counts(n_tok):
    _say(f"gather ragged n_tok={n_tok}")
    R = 512
    host_t, host_c = workloads.dense_tables(4242, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(n_tok)
    addr = rng.integers(0, R, size=(n_tok, 48)).astype(np.uint32)
    d_addr = torch.from_numpy(addr.view(np.int32)).cuda().view(torch.uint32)
    out = torch.full((n_tok + 1, 2, 256), 7.0, device="cuda")  # one guard token past the end
    lib().gather_reduce(plan, d_addr, out=out[:n_tok])
    torch.cuda.synchronize()
    want, abs_sum = oracle.gather_reduce(host_t, host_c, addr)
    res = out.cpu().numpy()
    assert_within_tolerance(res[:n_tok], want, abs_sum)
    assert np.all(res[n_tok] == 7.0), "wrote past the last token"


@pytest.mark.parametrize("key", [2, 3, 4, 5])
def test_lookup_workload_sampled(key):
    w = workloads.WORKLOADS[key]
    _say(f"lookup workload {key} ({w.name}) n_tok={w.n_tok} R={w.rows}")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    out = lib().gather_reduce(plan, addr)
    torch.cuda.synchronize()
    must = [w.prefix_len + k for k in range(4)] if w.prefix_len else []
    if w.n_seq > 1:
        must += [w.seq_len * s + j for s in (1, w.n_seq - 1) for j in (0, 1, w.seq_len - 1)]
    tokens = sample_tokens(w.n_tok, 8192, key, must)
    want_addr, want, abs_sum = oracle_sampled(ids, hist, w.rows, w.table_seed, tokens)
    assert np.array_equal(addr_to_host(addr), want_addr)
    got = out[torch.from_numpy(tokens).cuda()].cpu().numpy()
    assert_within_tolerance(got, want, abs_sum)


def test_address_revealing_tables_full_size():
    """Element q of module m equals the row read from sub-table 24m+q, on every token, exactly."""
    w = workloads.WORKLOADS[4]
    _say("address-revealing tables, full size, all tokens")
    t, c = device_tables(w.rows, w.table_seed)
    mark_buffer_dirty()
    for s in range(48):
        t[s].zero_()
        t[s][:, s % 24] = 0x38  # 1.0
        torch.arange(w.rows, out=c[s], dtype=torch.float32)  # exact below 2^24
    plan = lib().Plan(t, c)
    ids, hist = workloads.make_ids(w)
    addr = lib().hash(plan, *to_dev_ids(ids, hist))
    out = lib().gather_reduce(plan, addr)
    torch.cuda.synchronize()
    a = addr.view(torch.int32).to(torch.float32)  # rows < 2^24: exact
    for m in range(2):
        assert torch.equal(out[:, m, :24], a[:, 24 * m:24 * (m + 1)])
        assert not out[:, m, 24:].any()


def test_zero_tables_give_zero_full_size():
    w = workloads.WORKLOADS[4]
    _say("zero tables, full size")
    t, c = device_tables(w.rows, w.table_seed)
    mark_buffer_dirty()
    for s in range(48):
        t[s].zero_()
    plan = lib().Plan(t, c)
    ids, hist = workloads.make_ids(w)
    addr = lib().hash(plan, *to_dev_ids(ids, hist))
    out = lib().gather_reduce(plan, addr)
    torch.cuda.synchronize()
    assert not out.any()


def test_fp8_decode_exhaustive_on_device():
    """All 256 E4M3 codes through the real kernel against the oracle's decode table."""
    _say("fp8 decode exhaustive")
    host_t = [np.zeros((1, 256), np.uint8) for _ in range(48)]
    host_t[0][0] = np.arange(256, dtype=np.uint8)
    host_t[30][0] = np.arange(256, dtype=np.uint8)[::-1].copy()
    host_c = [np.ones(1, np.float32) for _ in range(48)]
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    ids = np.arange(8, dtype=np.int32).reshape(1, 8)
    addr = lib().hash(plan, *to_dev_ids(ids, None))
    out = lib().gather_reduce(plan, addr)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    dec = oracle.E4M3_TABLE
    for tok in range(8):
        assert np.array_equal(np.isnan(got[tok, 0]), np.isnan(dec))
        ok = ~np.isnan(dec)
        assert np.array_equal(got[tok, 0][ok], dec[ok])
        assert np.array_equal(got[tok, 1][ok[::-1]], dec[::-1][ok[::-1]])


def test_batch_invariance_bitwise():
    """A sequence's vectors do not depend on which sequences share its batch."""
    _say("batch invariance")
    R = 1 << 12
    host_t, host_c = workloads.dense_tables(555, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(1)
    a = rng.integers(0, 129280, size=(1, 700)).astype(np.int32)
    batch = rng.integers(0, 129280, size=(5, 700)).astype(np.int32)
    batch[3] = a[0]
    out_a = lib().gather_reduce(plan, lib().hash(plan, *to_dev_ids(a, None)))
    out_b = lib().gather_reduce(plan, lib().hash(plan, *to_dev_ids(batch, None)))
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b[3 * 700:4 * 700])


def test_error_paths_leave_output_untouched():
    _say("error paths")
    hg = lib()
    host_t, host_c = workloads.dense_tables(1, 16)
    t, c = small_device_tables(host_t, host_c)
    plan = hg.Plan(t, c)
    addr = torch.zeros((8, 48), dtype=torch.uint32, device="cuda")
    buf = torch.full((8 * 512 + 4,), 3.0, device="cuda")
    st = hg.lib().engram_gather_reduce(plan.handle, addr.data_ptr(), 8, None, None, None, buf.data_ptr() + 4, None)
    assert st == -1  # misaligned output
    with pytest.raises(ValueError):
        hg.gather_reduce(plan, addr[:, :47].contiguous())
    st = hg.lib().engram_gather_reduce(plan.handle, addr.data_ptr(), 8, buf.data_ptr(), None, None,
                                       buf.data_ptr(), None)
    assert st == -1  # partial dedup pointer set
    torch.cuda.synchronize()
    assert torch.all(buf == 3.0)


def test_probe_rows_equals_gather_with_unit_scales():
    _say("probe rows == gather with unit scales")
    R = 256
    host_t, _ = workloads.dense_tables(31, R)
    host_c = [np.ones(R, np.float32) for _ in range(48)]
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(4)
    addr = torch.from_numpy(rng.integers(0, R, size=(333, 48)).astype(np.int32)).cuda().view(torch.uint32)
    a = lib().gather_reduce(plan, addr)
    b = lib().probe_rows(plan, addr, torch.empty_like(a))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib().probe_read(t[0], sink)
    dst = torch.empty_like(t[1])
    lib().probe_copy(t[1], dst)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(dst, t[1])
