"""GPU parity with a vocabulary map and with prime row counts per sub-table."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (addr_to_host, assert_within_tolerance, big_buffer, lib, mark_buffer_dirty,
                         sample_tokens, to_dev_ids)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _map_plan(rows, vmap):
    t = torch.zeros((1, 256), dtype=torch.uint8, device="cuda")
    c = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_map = torch.from_numpy(vmap.view(np.int32)).cuda()
    return lib().Plan.from_pointers(rows, [t.data_ptr()] * 48, [c.data_ptr()] * 48, vocab_size=vmap.size,
                                    keep=(t, c, d_map), vocab_map_ptr=d_map.data_ptr())


@pytest.mark.parametrize("key", [2, 4, 5])
def test_hash_with_vocab_map_bit_exact(key):
    w = workloads.WORKLOADS[key]
    _say(f"hash with vocab map, workload {key}")
    ids, hist = workloads.make_ids(w)
    vmap = workloads.vocab_map(7)
    plan = _map_plan([w.rows] * 48, vmap)
    addr = lib().hash(plan, *to_dev_ids(ids, hist))
    torch.cuda.synchronize()
    want = oracle.hash_addresses(oracle.windows(ids, hist, vmap), oracle.multipliers(), [w.rows] * 48)
    assert np.array_equal(addr_to_host(addr), want)


def test_prime_rows_lookup_sampled():
    """Per-sub-table prime row counts (bucket ranges of prime size), with a vocab map, full-size tables."""
    w = workloads.WORKLOADS[4]
    _say("prime rows + vocab map, full-size tables")
    rows = workloads.prime_rows()
    tabs, scs = big_buffer()
    mark_buffer_dirty()
    t = [tabs[s, :rows[s]] for s in range(48)]
    c = [scs[s, :rows[s]] for s in range(48)]
    lib().synth_fill(t, c, 4321)
    vmap = workloads.vocab_map(7)
    d_map = torch.from_numpy(vmap.view(np.int32)).cuda()
    plan = lib().Plan(t, c, vocab_map=d_map)
    ids, hist = workloads.make_ids(w)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    out = lib().gather_reduce(plan, addr)
    fused = lib().lookup(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    want_addr = oracle.hash_addresses(oracle.windows(ids, hist, vmap), oracle.multipliers(), rows)
    assert np.array_equal(addr_to_host(addr), want_addr)
    assert torch.equal(fused, out)
    tokens = sample_tokens(w.n_tok, 4096, 5)
    host = workloads.SparseHostTables(4321, 1 << 24)  # row contents depend on (seed, sub-table, row) only
    try:
        host.materialise(want_addr[tokens])
        want, abs_sum = oracle.gather_reduce(host.tables, host.scales, want_addr[tokens])
    finally:
        host.close()
    assert_within_tolerance(out[torch.from_numpy(tokens).cuda()].cpu().numpy(), want, abs_sum)
