"""A seeded sweep over the lookup paths against the oracle.  Each case draws a batch shape, row counts per
sub-table (powers of two, one odd count, or a mix that includes 1-row sub-tables), a scale format, history or
none, a vocabulary map or none, a hash seed and an id range (from a handful of ids, so windows repeat, to the
whole vocabulary).  Cases 16 and up are batches of 8,192 tokens or more, where the batch-order paths share one
gather among the waves of a block with equal addresses; their sequences also share a prefix of random length.
Every token's addresses must equal the oracle's bit for bit, and every memory vector must lie
within 1e-5 x sum|terms| of the oracle, through every path that computes it: engram_hash + engram_gather_reduce,
engram_lookup, engram_gather_reduce_batched, and the dedup-mode gather and lookup over engram_dedup's groups.
The paths share one summation order, so they must also agree with each other bitwise."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import addr_to_host, assert_within_tolerance, lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _rows(kind, rng):
    if kind == 0:  # one power of two for every sub-table
        return [1 << int(rng.integers(4, 13))] * 48
    if kind == 1:  # one odd count for every sub-table
        return [int(rng.integers(500, 3000)) | 1] * 48
    rows = [int(x) for x in rng.integers(1, 4097, size=48)]  # a different count per sub-table
    if kind == 3:
        rows[int(rng.integers(0, 48))] = 1
        rows[int(rng.integers(0, 48))] = 2
        rows[int(rng.integers(0, 48))] = 4096
    return rows


def _tables(seed, rows, fmt):
    host_t, host_c = [], []
    for s, r in enumerate(rows):
        codes, sc = workloads.table_range(seed, s, 0, r)
        host_t.append(codes)
        host_c.append(sc if fmt == "f32_row" else workloads.e8m0_range(seed, s, 0, r))
    dev_t = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in host_t]
    dev_c = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in host_c]
    return host_t, host_c, dev_t, dev_c


@pytest.mark.parametrize("case", range(24))
def test_lookup_paths_random_cases(case):
    rng = np.random.default_rng(7000 + case)
    large = case >= 16
    if large:
        n_seq = int((8, 12, 16, 24, 57, 64, 9, 33)[case - 16])
        seq_len = -(-int(rng.integers(8192, 12000)) // n_seq)
    else:
        n_seq = int(rng.integers(1, 9))
        seq_len = int(rng.integers(1, 400))
    fmt = ("f32_row", "e8m0_block32")[case % 2]
    rows = _rows((case // 2) % 4, rng)
    with_hist = bool(rng.integers(0, 2))
    use_map = case % 3 == 0
    hash_seed = oracle.DEFAULT_HASH_SEED if case % 4 == 0 else int(rng.integers(0, 1 << 63, dtype=np.uint64))
    vocab = workloads.VOCAB if use_map else 0
    hi = int([3, 60, 129280, 1 << 31][int(rng.integers(0, 4))])
    if use_map:
        hi = min(hi, workloads.VOCAB)
    _say(f"sweep case {case}: {n_seq}x{seq_len} {fmt} rows[0]={rows[0]} hist={with_hist} map={use_map} ids<{hi}")
    ids = rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    if large:  # every sequence starts with the first one's prefix
        prefix = int(rng.integers(0, seq_len + 1))
        ids[:, :prefix] = ids[0, :prefix]
    hist = rng.integers(0, hi, size=(n_seq, 3), dtype=np.int64).astype(np.int32) if with_hist else None
    vmap = workloads.vocab_map(100 + case) if use_map else None

    host_t, host_c, dev_t, dev_c = _tables(500 + case, rows, fmt)
    d_map = torch.from_numpy(vmap.view(np.int32)).cuda() if use_map else None
    plan = lib().Plan(dev_t, dev_c, hash_seed=hash_seed, vocab_size=vocab, scale_format=fmt, vocab_map=d_map)
    d_ids = torch.from_numpy(ids).cuda()
    d_hist = torch.from_numpy(hist).cuda() if with_hist else None

    want_addr, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, rows, hash_seed, fmt, vmap)
    addr = lib().hash(plan, d_ids, d_hist)
    groups = lib().dedup(plan, d_ids, d_hist)
    outs = {
        "two calls": lib().gather_reduce(plan, addr),
        "fused": lib().lookup(plan, d_ids, d_hist),
        "batch order": lib().gather_reduce_batched(plan, addr, n_seq),
        "dedup gather": lib().gather_reduce(plan, addr, groups=groups),
        "dedup lookup": lib().lookup(plan, d_ids, d_hist, groups=groups),
    }
    torch.cuda.synchronize()
    assert np.array_equal(addr_to_host(addr), want_addr)
    ref = outs["two calls"]
    for name, out in outs.items():
        assert_within_tolerance(out.cpu().numpy(), want, abs_sum)
        assert torch.equal(torch.nan_to_num(out, nan=7.0), torch.nan_to_num(ref, nan=7.0)), name
