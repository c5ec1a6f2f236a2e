"""engram_gather_reduce_batched and the batched engram_lookup, which visit a batch in tiles of positions: against
the oracle (full-size shared-prefix batch, a ragged batch, both sides of the 2^24-item launch split), and bitwise
against the flat gather for every shape (ragged last tiles, sequences shorter than a tile, one sequence) and both
scale formats."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (addr_to_host, assert_within_tolerance, batch_sample, device_tables, lib, oracle_sampled,
                         small_device_tables, to_dev_ids, unwritten_tokens)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("fmt", ["f32_row", "e8m0_block32"])
@pytest.mark.parametrize("n_seq,seq_len,shared", [
    (1, 1000, 0), (3, 5, 0), (5, 77, 30), (2, 64, 64), (7, 129, 0), (64, 1, 0),
    # below 8,192 tokens (no sharing between waves): 2 or 4 sequences per
    # block with idle waves or idle positions in a narrow tile
    (9, 70, 40), (33, 67, 50), (6, 3, 3), (10, 67, 20),
    # 8,192 tokens and more (waves with equal addresses share one gather):
    # 8 sequences per block (8-wave blocks); 8 per block with seven idle
    # waves; 2 per block with one idle; 4 per block with three idle; idle
    # positions in a narrow last tile; every sequence equal
    (64, 300, 128), (24, 350, 100), (57, 150, 60), (9, 1000, 400), (33, 260, 100), (10, 835, 300),
    (4, 2050, 2050),
])
def test_batched_equals_flat(fmt, n_seq, seq_len, shared):
    _say(f"batched gather {n_seq}x{seq_len} shared={shared} {fmt}")
    R = 4096
    host_t, host_c = workloads.dense_tables(31, R, fmt)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=fmt)
    rng = np.random.default_rng(n_seq * 1000 + seq_len)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len)).astype(np.int32)
    if shared:
        ids[:, :shared] = ids[0, :shared]
    d_ids, _ = to_dev_ids(ids, None)
    addr = lib().hash(plan, d_ids)
    flat = lib().gather_reduce(plan, addr)
    batched = torch.full_like(flat, float("nan"))
    lib().gather_reduce_batched(plan, addr, n_seq, out=batched)
    fused = lib().lookup(plan, d_ids)
    torch.cuda.synchronize()
    assert torch.equal(batched, flat)
    assert torch.equal(fused, flat)


@pytest.mark.parametrize("n_seq", [8, 10, 16])
def test_batched_partial_sharing_within_blocks(n_seq):
    """Sequences equal to a later, not the first, sequence of their block, and
    equal over part of their length only: every wave must take the sum of the
    first equal wave or gather its own."""
    _say(f"batched gather + fused lookup, {n_seq} sequences with scattered duplicates")
    t, c = small_device_tables(*workloads.dense_tables(32, 4096, "f32_row"))
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(700 + n_seq)
    ids = rng.integers(0, 129280, size=(n_seq, 1100)).astype(np.int32)  # >= 8,192 tokens: sharing on
    ids[2] = ids[1]
    ids[3, :550] = ids[0, :550]
    ids[7, 300:] = ids[5, 300:]
    ids[6, ::2] = ids[4, ::2]
    if n_seq >= 16:
        ids[15] = ids[9]
        ids[12, 700:] = ids[0, 700:]
    d_ids, _ = to_dev_ids(ids, None)
    addr = lib().hash(plan, d_ids)
    flat = lib().gather_reduce(plan, addr)
    batched = torch.full_like(flat, float("nan"))
    lib().gather_reduce_batched(plan, addr, n_seq, out=batched)
    fused = torch.full_like(flat, float("nan"))
    lib().lookup(plan, d_ids, out=fused)
    torch.cuda.synchronize()
    assert torch.equal(batched, flat)
    assert torch.equal(fused, flat)


def _batched_against_oracle(ids, hist, rows, seed, sample, what):
    n_seq, seq_len = ids.shape
    t, c = device_tables(rows, seed)
    plan = lib().Plan(t, c)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    out = torch.full((n_seq * seq_len, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().gather_reduce_batched(plan, addr, n_seq, out=out)
    idx = torch.from_numpy(sample).cuda()
    got = out[idx].cpu().numpy()
    unwritten = unwritten_tokens(out)
    got_addr = addr_to_host(addr)
    out.fill_(float("nan"))
    lib().lookup(plan, d_ids, d_hist, out=out)
    got_fused = out[idx].cpu().numpy()
    unwritten_fused = unwritten_tokens(out)
    torch.cuda.synchronize()
    del out, addr
    torch.cuda.empty_cache()
    assert unwritten == 0, f"{unwritten} tokens the batched gather never wrote"
    assert unwritten_fused == 0, f"{unwritten_fused} tokens the fused lookup never wrote"
    _say(f"oracle on {sample.size} sampled tokens ({what})")
    want_addr, want, abs_sum = oracle_sampled(ids, hist, rows, seed, sample)
    assert np.array_equal(got_addr, want_addr)
    assert_within_tolerance(got, want, abs_sum)
    assert_within_tolerance(got_fused, want, abs_sum)
    assert np.array_equal(got_fused, got)


def test_batched_shared_prefix_full_size_against_oracle():
    """The shared-prefix batch (64 x (4,096 shared + 4,096 own), 48 x 2^24-row tables): the batch-order gather and
    the batch-order fused lookup against the oracle on 8,192 sampled tokens, including positions 0-3, 63-65,
    4,095-4,099 and the last one of several sequences."""
    w = workloads.WORKLOADS[5]
    _say(f"batched gather + fused lookup vs oracle, workload 5 n_tok={w.n_tok}")
    ids, hist = workloads.make_ids(w)
    sample = batch_sample(w.n_seq, w.seq_len, 8192, 55, seqs=(0, 1, 2, 31, 62, 63),
                          positions=(127, 128, 4095, 4096, 4097, 4098, 4099, 8127, 8128))
    _batched_against_oracle(ids, hist, w.rows, w.table_seed, sample, "workload 5")


def test_batched_ragged_full_size_against_oracle():
    """7 sequences of 4,133 positions (a 37-position last tile) sharing a 1,000-id prefix, on the full-size
    tables: the batch-order paths against the oracle on 8,192 sampled tokens."""
    w = workloads.WORKLOADS[5]
    n_seq, seq_len, shared = 7, 4133, 1000
    _say(f"batched gather + fused lookup vs oracle, {n_seq} x {seq_len}, ragged last tile")
    rng = np.random.default_rng(4133)
    ids = workloads.zipf_ids(rng, n_seq * seq_len).reshape(n_seq, seq_len)
    ids[:, :shared] = ids[0, :shared]
    sample = batch_sample(n_seq, seq_len, 8192, 56, seqs=tuple(range(n_seq)),
                          positions=(999, 1000, 1001, 4095, 4096, 4097, 4131))
    _batched_against_oracle(ids, None, w.rows, w.table_seed, sample, "ragged batch")


def test_batched_across_the_chunk_boundary():
    """Two sequences of 2^23 + 40 tokens: the batched gather splits its grid at 2^24 items, where the last,
    40-position tile begins.  The output starts as NaN; tokens on both sides of the split (the last 1,200
    positions of each sequence, the first 130, and 4,000 at random) are checked against the oracle and bitwise
    against the flat gather, and no token is left unwritten."""
    n_seq, seq_len = 2, (1 << 23) + 40
    _say(f"batched gather, {n_seq} x {seq_len} tokens")
    R = 512
    host_t, host_c = workloads.dense_tables(810, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(26)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = n_seq * seq_len
    sample = np.unique(np.concatenate([
        np.arange(0, 130), np.arange(seq_len - 1200, seq_len + 130), np.arange(n_tok - 1200, n_tok),
        rng.integers(0, n_tok, 4000)]))
    idx = torch.from_numpy(sample).cuda()
    addr = lib().hash(plan, d_ids)
    out = torch.full((n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().gather_reduce_batched(plan, addr, n_seq, out=out)
    batched_sample = out[idx].cpu().numpy()
    unwritten = unwritten_tokens(out)
    out.fill_(float("nan"))
    lib().gather_reduce(plan, addr, out=out)
    flat_sample = out[idx].cpu().numpy()
    got_addr = addr.view(torch.int32)[idx].cpu().numpy().view(np.uint32)
    torch.cuda.synchronize()
    del addr, out
    torch.cuda.empty_cache()
    assert unwritten == 0
    want_addr = oracle.hash_addresses(oracle.windows(ids)[sample], oracle.multipliers(), [R] * 48)
    assert np.array_equal(got_addr, want_addr)
    want, abs_sum = oracle.gather_reduce(host_t, host_c, want_addr)
    assert_within_tolerance(batched_sample, want, abs_sum)
    assert np.array_equal(batched_sample, flat_sample)


@pytest.mark.parametrize("route", ["lookup", "gather_batched", "lookup_dedup", "gather_dedup"])
def test_batch_invariance_of_the_batch_paths(route):
    """A sequence's vectors are bitwise the same whichever sequences share its batch, also on the paths where the
    batch changes the visiting order (tiles of positions across sequences) or the work itself (dedup groups that
    span sequences): the sequence alone, by the flat two calls, against the same sequence as row 4 of a 6-sequence
    batch whose row 1 shares its first 300 ids and whose row 5 repeats it whole.  The batch holds 8,400 tokens,
    enough for the batch order to share sums between the waves of a block."""
    _say(f"batch invariance through {route}")
    R = 4096
    host_t, host_c = workloads.dense_tables(557, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, vocab_size=workloads.VOCAB)
    rng = np.random.default_rng(3)
    L = 1400
    a = workloads.zipf_ids(rng, L).reshape(1, L)
    batch = workloads.zipf_ids(rng, 6 * L).reshape(6, L)
    batch[4] = a[0]
    batch[5] = a[0]
    batch[1, :300] = a[0, :300]
    alone = lib().gather_reduce(plan, lib().hash(plan, *to_dev_ids(a, None)))
    d_ids, _ = to_dev_ids(batch, None)
    out = torch.full((batch.size, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    if route == "lookup":
        lib().lookup(plan, d_ids, out=out)
    elif route == "gather_batched":
        lib().gather_reduce_batched(plan, lib().hash(plan, d_ids), 6, out=out)
    elif route == "lookup_dedup":
        lib().lookup(plan, d_ids, out=out, groups=lib().dedup(plan, d_ids))
    else:
        lib().gather_reduce(plan, lib().hash(plan, d_ids), out=out, groups=lib().dedup(plan, d_ids))
    torch.cuda.synchronize()
    assert torch.equal(out[4 * L:5 * L], alone)
    assert torch.equal(out[5 * L:6 * L], alone)


def test_sharing_paths_graph_replay_matches_eager():
    """hash + engram_gather_reduce_batched + engram_lookup on a 16 x 640 batch (10,240 tokens: 8 sequences per
    block, waves with equal addresses share one gather) capture into one HIP graph; each replay, on new ids with a
    shared prefix of a new length, matches the eager flat gather bitwise and the oracle within tolerance."""
    _say("batch-order sharing paths in a hip graph")
    n_seq, seq_len, R = 16, 640, 4096
    host_t, host_c = workloads.dense_tables(33, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(34)

    def draw():
        ids = workloads.zipf_ids(rng, n_seq * seq_len).reshape(n_seq, seq_len)
        prefix = int(rng.integers(0, seq_len + 1))
        ids[:, :prefix] = ids[0, :prefix]
        return ids

    ids = draw()
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = n_seq * seq_len
    addr = torch.empty((n_tok, 48), dtype=torch.uint32, device="cuda")
    out_b = torch.empty((n_tok, 2, 256), dtype=torch.float32, device="cuda")
    out_f = torch.empty_like(out_b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the side stream, as capture requires
        lib().hash(plan, d_ids, out=addr)
        lib().gather_reduce_batched(plan, addr, n_seq, out=out_b)
        lib().lookup(plan, d_ids, out=out_f)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib().hash(plan, d_ids, out=addr)
        lib().gather_reduce_batched(plan, addr, n_seq, out=out_b)
        lib().lookup(plan, d_ids, out=out_f)
    for rep in range(4):
        ids = draw()
        d_ids.copy_(torch.from_numpy(ids))
        out_b.fill_(float("nan"))
        out_f.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        eager = lib().gather_reduce(plan, lib().hash(plan, d_ids))
        torch.cuda.synchronize()
        assert torch.equal(out_b, eager), rep
        assert torch.equal(out_f, eager), rep
        sample = np.concatenate([np.arange(0, 70), rng.integers(0, n_tok, size=400), np.arange(n_tok - 70, n_tok)])
        _, want, abs_sum = oracle.lookup(ids, None, host_t, host_c, [R] * 48)
        assert_within_tolerance(out_b.cpu().numpy()[sample], want[sample], abs_sum[sample])


@pytest.mark.parametrize("n_seq,seq_len", [(8200, 1), (4100, 2), (2731, 3)])
def test_sharing_with_history_windows(n_seq, seq_len):
    """Large batches of very short sequences (a big decode or speculative step): every window reads the caller's
    history, and the batch holds 8,192 tokens or more, so waves with equal addresses share one gather.  Ids and
    histories come from a few values and repeat, so many windows are equal.  The batch-order gather and the fused
    lookup must equal the flat gather bitwise and the oracle within tolerance on every token."""
    _say(f"sharing with history windows, {n_seq} x {seq_len}")
    R = 4096
    host_t, host_c = workloads.dense_tables(35, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(36 + seq_len)
    ids = rng.integers(0, 5, size=(n_seq, seq_len)).astype(np.int32)
    hist = rng.integers(0, 5, size=(n_seq, 3)).astype(np.int32)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    flat = lib().gather_reduce(plan, addr)
    batched = torch.full_like(flat, float("nan"))
    lib().gather_reduce_batched(plan, addr, n_seq, out=batched)
    fused = torch.full_like(flat, float("nan"))
    lib().lookup(plan, d_ids, d_hist, out=fused)
    torch.cuda.synchronize()
    assert torch.equal(batched, flat)
    assert torch.equal(fused, flat)
    want_addr, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, [R] * 48)
    assert np.array_equal(addr_to_host(addr), want_addr)
    assert_within_tolerance(flat.cpu().numpy(), want, abs_sum)
