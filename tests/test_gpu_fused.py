"""Fused lookup (engram_lookup) against the two-call path and the oracle; HIP-graph replay."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import assert_within_tolerance, device_tables, lib, small_device_tables, to_dev_ids, unwritten_tokens

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def test_fused_tiny_against_oracle():
    w = workloads.WORKLOADS[1]
    _say("fused lookup, tiny workload, all tokens vs oracle")
    ids, hist = workloads.make_ids(w)
    host_t, host_c = workloads.dense_tables(w.table_seed, w.rows)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    out = lib().lookup(plan, *to_dev_ids(ids, hist))
    torch.cuda.synchronize()
    _, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, [w.rows] * 48)
    assert_within_tolerance(out.cpu().numpy(), want, abs_sum)


@pytest.mark.parametrize("key", [2, 3, 4, 5])
def test_fused_equals_two_calls_workloads(key):
    w = workloads.WORKLOADS[key]
    _say(f"fused == hash + gather, workload {key}")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c)
    d_ids, d_hist = to_dev_ids(ids, hist)
    two = lib().gather_reduce(plan, lib().hash(plan, d_ids, d_hist))
    fused = torch.full_like(two, float("nan"))
    lib().lookup(plan, d_ids, d_hist, out=fused)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)


@pytest.mark.parametrize("n_seq,seq_len,with_hist,rows", [
    (1, 1, True, 1000003), (3, 5, True, 4099), (2, 333, False, 1 << 16), (5, 77, True, 65537), (1, 1, False, 1),
])
def test_fused_equals_two_calls_shapes(n_seq, seq_len, with_hist, rows):
    _say(f"fused shapes {n_seq}x{seq_len} hist={with_hist} R={rows}")
    rng = np.random.default_rng(rows + seq_len)
    t, c = device_tables(rows, 3000 + rows % 1000)
    plan = lib().Plan(t, c)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len)).astype(np.int32)
    hist = rng.integers(0, 129280, size=(n_seq, 3)).astype(np.int32) if with_hist else None
    d_ids, d_hist = to_dev_ids(ids, hist)
    two = lib().gather_reduce(plan, lib().hash(plan, d_ids, d_hist))
    fused = lib().lookup(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)


def test_graph_replay_matches_eager():
    """The stream-ordered calls capture into a HIP graph; every replay matches eager results."""
    _say("hip graph capture and replay")
    R = 4096
    host_t, host_c = workloads.dense_tables(9, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(8)
    ids_a = rng.integers(0, 129280, size=(64, 1)).astype(np.int32)
    hist_a = rng.integers(0, 129280, size=(64, 3)).astype(np.int32)
    d_ids, d_hist = to_dev_ids(ids_a, hist_a)
    addr = torch.empty((64, 48), dtype=torch.uint32, device="cuda")
    out = torch.empty((64, 2, 256), dtype=torch.float32, device="cuda")
    out_f = torch.empty_like(out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the side stream, as capture requires
        lib().hash(plan, d_ids, d_hist, out=addr)
        lib().gather_reduce(plan, addr, out=out)
        lib().lookup(plan, d_ids, d_hist, out=out_f)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib().hash(plan, d_ids, d_hist, out=addr)
        lib().gather_reduce(plan, addr, out=out)
        lib().lookup(plan, d_ids, d_hist, out=out_f)
    for rep in range(4):
        new_ids = rng.integers(0, 129280, size=(64, 1)).astype(np.int32)
        new_hist = rng.integers(0, 129280, size=(64, 3)).astype(np.int32)
        d_ids.copy_(torch.from_numpy(new_ids))
        d_hist.copy_(torch.from_numpy(new_hist))
        out.zero_()
        out_f.zero_()
        g.replay()
        torch.cuda.synchronize()
        eager = lib().gather_reduce(plan, lib().hash(plan, d_ids, d_hist))
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        assert torch.equal(out_f, eager), rep
        _, want, abs_sum = oracle.lookup(new_ids, new_hist, host_t, host_c, [R] * 48)
        assert_within_tolerance(out.cpu().numpy(), want, abs_sum)


def test_launch_chunk_boundary():
    """More than 2^24 tokens: the gather and the fused lookup split their grids at 2^24 items.  Each output starts
    as NaN; 2,400 tokens on both sides of the split, the first and last tokens and 2,000 at random are checked
    against the oracle, the fused result bitwise against the gather's, and no token may stay unwritten."""
    n_tok = (1 << 24) + 37
    _say(f"chunk boundary, {n_tok} tokens (3.2 GB addresses, 34 GB output)")
    R = 512
    host_t, host_c = workloads.dense_tables(808, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(24)
    ids = rng.integers(0, 129280, size=(1, n_tok), dtype=np.int64).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    tokens = np.unique(np.concatenate([np.arange(0, 64), np.arange((1 << 24) - 2400, n_tok),
                                       rng.integers(0, n_tok, 2000)]))
    idx = torch.from_numpy(tokens).cuda()
    addr = lib().hash(plan, d_ids)
    out = torch.full((n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().gather_reduce(plan, addr, out=out)
    got = out[idx].cpu().numpy()
    unwritten = unwritten_tokens(out)
    got_addr = addr.view(torch.int32)[idx].cpu().numpy().view(np.uint32)
    out.fill_(float("nan"))
    lib().lookup(plan, d_ids, out=out)
    got_fused = out[idx].cpu().numpy()
    unwritten_fused = unwritten_tokens(out)
    torch.cuda.synchronize()
    del addr, out
    torch.cuda.empty_cache()
    assert unwritten == 0 and unwritten_fused == 0, (unwritten, unwritten_fused)
    win = oracle.windows(ids)[tokens]
    want_addr = oracle.hash_addresses(win, oracle.multipliers(), [R] * 48)
    assert np.array_equal(got_addr, want_addr)
    want, abs_sum = oracle.gather_reduce(host_t, host_c, want_addr)
    assert_within_tolerance(got, want, abs_sum)
    assert_within_tolerance(got_fused, want, abs_sum)
    assert np.array_equal(got_fused, got)


def test_batched_order_across_the_chunk_boundary():
    """Two sequences of 2^23 + 40 tokens: the fused lookup visits them in 64-position tiles and splits its grid at
    2^24 items, which is where the last, 40-position tile begins.  The output starts as NaN; the last 1,200
    positions of each sequence (both sides of the split), the first 130 and 4,000 at random are checked against
    the oracle and bitwise against the two-call path, and no token may stay unwritten."""
    n_seq, seq_len = 2, (1 << 23) + 40
    _say(f"fused batched order, {n_seq} x {seq_len} tokens")
    R = 512
    host_t, host_c = workloads.dense_tables(809, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(25)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = n_seq * seq_len
    sample = np.unique(np.concatenate([
        np.arange(0, 130), np.arange(seq_len - 1200, seq_len + 130), np.arange(n_tok - 1200, n_tok),
        rng.integers(0, n_tok, 4000)]))
    idx = torch.from_numpy(sample).cuda()
    out = torch.full((n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().lookup(plan, d_ids, out=out)
    fused_sample = out[idx].cpu().numpy()
    unwritten = unwritten_tokens(out)
    addr = lib().hash(plan, d_ids)
    out.fill_(float("nan"))
    lib().gather_reduce(plan, addr, out=out)
    two_sample = out[idx].cpu().numpy()
    torch.cuda.synchronize()
    del addr, out
    torch.cuda.empty_cache()
    assert unwritten == 0
    want_addr = oracle.hash_addresses(oracle.windows(ids)[sample], oracle.multipliers(), [R] * 48)
    want, abs_sum = oracle.gather_reduce(host_t, host_c, want_addr)
    assert_within_tolerance(fused_sample, want, abs_sum)
    assert np.array_equal(fused_sample, two_sample)


def test_one_plan_on_two_streams():
    """A plan is immutable: concurrent calls on two streams give the sequential results (the 4 x 3,000-token
    batches are large enough for the batch-order paths to share gathers within a block)."""
    _say("one plan, two streams")
    R = 4096
    host_t, host_c = workloads.dense_tables(10, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, vocab_size=129280)
    rng = np.random.default_rng(31)
    batches = [rng.integers(0, 129280, size=(4, 3000)).astype(np.int32) for _ in range(2)]
    d = [to_dev_ids(b, None)[0] for b in batches]
    want = [lib().gather_reduce(plan, lib().hash(plan, x)) for x in d]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(want[0]) for _ in range(2)]
    fused = [torch.empty_like(want[0]) for _ in range(2)]
    groups_out = [torch.empty_like(want[0]) for _ in range(2)]
    batched_out = [torch.empty_like(want[0]) for _ in range(2)]
    for rep in range(3):
        for i, s in enumerate(streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                a = lib().hash(plan, d[i], stream=s)
                lib().gather_reduce(plan, a, out=outs[i], stream=s)
                lib().lookup(plan, d[i], out=fused[i], stream=s)
                g = lib().dedup(plan, d[i], stream=s)
                lib().gather_reduce(plan, a, out=groups_out[i], groups=g, stream=s)
                lib().gather_reduce_batched(plan, a, 4, out=batched_out[i], stream=s)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], want[i]), (rep, i)
            assert torch.equal(fused[i], want[i]), (rep, i)
            assert torch.equal(groups_out[i], want[i]), (rep, i)
            assert torch.equal(batched_out[i], want[i]), (rep, i)
