"""engram_lookup_dedup, the fused lookup over the groups engram_dedup wrote: against the oracle (small tables in
every plan variant; the decode, prefill and shared-prefix workloads at full size), bitwise against the direct fused
lookup and the two-call path, with failed or out-of-range groups, and under HIP-graph replay."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (assert_within_tolerance, batch_sample, device_tables, lib, oracle_sampled,
                         small_device_tables, to_dev_ids, unwritten_tokens)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _new_groups(n_tok):
    return lib().Groups(torch.empty(n_tok, dtype=torch.int32, device="cuda"),
                        torch.empty(n_tok + 1, dtype=torch.int32, device="cuda"),
                        torch.empty(1, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("fmt", ["f32_row", "e8m0_block32"])
@pytest.mark.parametrize("variant", ["pow2", "prime_rows", "vocab_map", "history"])
@pytest.mark.parametrize("n_seq,seq_len", [(1, 1), (7, 333), (64, 65), (3, 2000)])
def test_lookup_dedup_small_against_oracle(fmt, variant, n_seq, seq_len):
    """Ids from a handful of values, so that many windows repeat; every token against the oracle, and bitwise
    equal to the direct fused lookup and to hash + dedup-mode gather."""
    _say(f"lookup dedup {n_seq}x{seq_len} {variant} {fmt}")
    R = 4096
    host_t, host_c = workloads.dense_tables(90 + n_seq, R, fmt)
    rows = [R] * 48
    if variant == "prime_rows":
        rows = workloads.prime_rows(48, R)
        host_t = [host_t[s][:rows[s]] for s in range(48)]
        host_c = [host_c[s][:rows[s]] for s in range(48)]
    t, c = small_device_tables(host_t, host_c)
    rng = np.random.default_rng(n_seq * 7 + seq_len)
    vmap = hist = None
    if variant == "vocab_map":
        vmap = workloads.vocab_map(7)
        plan = lib().Plan(t, c, scale_format=fmt, vocab_map=torch.from_numpy(vmap.view(np.int32)).cuda())
        ids = rng.choice(np.array([0, 5, 99091, 129279], np.int32), size=(n_seq, seq_len))
    else:
        plan = lib().Plan(t, c, scale_format=fmt, vocab_size=7)
        ids = rng.integers(0, 7, size=(n_seq, seq_len)).astype(np.int32)
        if variant == "history":
            hist = rng.integers(0, 7, size=(n_seq, 3)).astype(np.int32)
    d_ids, d_hist = to_dev_ids(ids, hist)
    groups = lib().dedup(plan, d_ids, d_hist)
    n_tok = ids.size
    out = torch.full((n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().lookup(plan, d_ids, d_hist, out=out, groups=groups)
    direct = lib().lookup(plan, d_ids, d_hist)
    addr = lib().hash(plan, d_ids, d_hist)
    two_call = torch.full_like(out, float("nan"))
    lib().gather_reduce(plan, addr, out=two_call, groups=groups)
    torch.cuda.synchronize()
    nu = int(groups.n_unique.item())
    _, _, want_nu = oracle.dedup(oracle.windows(ids, hist))
    assert nu == want_nu
    _, want, abs_sum = oracle.lookup(ids, hist, host_t, host_c, rows, scale_format=fmt, vocab_map=vmap)
    got = out.cpu().numpy()
    assert_within_tolerance(got.reshape(n_tok, 2, 256), want, abs_sum)
    assert torch.equal(out, direct)
    assert torch.equal(out, two_call)


def test_lookup_dedup_shared_prefix_full_size_against_oracle():
    """The shared-prefix batch (64 x (4,096 shared + 4,096 own), 48 x 2^24-row tables): every token written, the
    result bitwise equal to the batch-order direct lookup, and 8,192 sampled tokens (positions 0-3, 63-65,
    4,095-4,099 and the last of several sequences among them) against the oracle."""
    w = workloads.WORKLOADS[5]
    _say(f"lookup dedup vs oracle, workload 5 n_tok={w.n_tok}")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c, vocab_size=workloads.VOCAB)
    d_ids, d_hist = to_dev_ids(ids, hist)
    groups = lib().dedup(plan, d_ids, d_hist)
    out = torch.full((w.n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().lookup(plan, d_ids, d_hist, out=out, groups=groups)
    unwritten = unwritten_tokens(out)
    direct = lib().lookup(plan, d_ids, d_hist)
    same = torch.equal(out, direct)
    sample = batch_sample(w.n_seq, w.seq_len, 8192, 57, seqs=(0, 1, 2, 31, 62, 63),
                          positions=(127, 128, 4095, 4096, 4097, 4098, 4099, 8127, 8128))
    got = out[torch.from_numpy(sample).cuda()].cpu().numpy()
    nu = int(groups.n_unique.item())
    torch.cuda.synchronize()
    del out, direct
    torch.cuda.empty_cache()
    _say(f"n_unique={nu}")
    assert unwritten == 0, f"{unwritten} tokens never written"
    assert same
    assert nu < w.n_tok * 0.6
    _, want, abs_sum = oracle_sampled(ids, hist, w.rows, w.table_seed, sample)
    assert_within_tolerance(got, want, abs_sum)


@pytest.mark.parametrize("key", [2, 3])
def test_lookup_dedup_workloads_against_oracle(key):
    """Decode (64 sequences x 1 token after a 3-token history, 2^20-row tables) and the 32K prefill (2^22-row
    tables): every token written, bitwise the direct fused lookup, and against the oracle on all tokens (decode)
    or 8,192 sampled ones (prefill)."""
    w = workloads.WORKLOADS[key]
    _say(f"lookup dedup, workload {key} n_tok={w.n_tok}")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c, vocab_size=workloads.VOCAB)
    d_ids, d_hist = to_dev_ids(ids, hist)
    groups = lib().dedup(plan, d_ids, d_hist)
    out = torch.full((w.n_tok, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().lookup(plan, d_ids, d_hist, out=out, groups=groups)
    direct = lib().lookup(plan, d_ids, d_hist)
    torch.cuda.synchronize()
    assert unwritten_tokens(out) == 0
    assert torch.equal(out, direct)
    assert int(groups.n_unique.item()) == oracle.dedup(oracle.windows(ids, hist))[2]
    sample = batch_sample(w.n_seq, w.seq_len, 8192, 58 + key, seqs=(0, 1, w.n_seq - 1))
    got = out[torch.from_numpy(sample).cuda()].cpu().numpy()
    _, want, abs_sum = oracle_sampled(ids, hist, w.rows, w.table_seed, sample)
    assert_within_tolerance(got, want, abs_sum)


def _small_plan(seed, R=1024):
    host_t, host_c = workloads.dense_tables(seed, R)
    t, c = small_device_tables(host_t, host_c)
    return lib().Plan(t, c, vocab_size=129280)


def test_lookup_dedup_failed_groups_write_nothing():
    """n_unique = -1 (what a dedup call that gave up reports): the fused dedup lookup writes no token."""
    _say("lookup dedup with n_unique = -1")
    plan = _small_plan(91)
    rng = np.random.default_rng(91)
    ids = rng.integers(0, 50, size=(4, 500)).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    groups = lib().dedup(plan, d_ids)
    groups.n_unique.fill_(-1)
    out = torch.full((ids.size, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    lib().lookup(plan, d_ids, out=out, groups=groups)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())


def test_lookup_dedup_skips_out_of_range_entries():
    """A perm entry outside [0, n_tok) is skipped: a group whose first entry is bad is not looked up (its members
    stay unwritten), a bad later entry drops only that member; every other token equals the direct result."""
    _say("lookup dedup with planted perm entries out of range")
    plan = _small_plan(92)
    rng = np.random.default_rng(92)
    ids = rng.integers(0, 4, size=(2, 700)).astype(np.int32)  # 256 possible windows: many groups of several
    n_tok = ids.size
    d_ids, _ = to_dev_ids(ids, None)
    groups = lib().dedup(plan, d_ids)
    direct = lib().lookup(plan, d_ids)
    torch.cuda.synchronize()
    perm = groups.perm.cpu().numpy()
    off = groups.offsets.cpu().numpy()
    nu = int(groups.n_unique.item())
    sizes = np.diff(off[:nu + 1])
    u, v = [int(g) for g in np.flatnonzero(sizes >= 2)[:2]]
    lost = list(perm[off[u]:off[u + 1]]) + [int(perm[off[v] + 1])]
    bad = perm.copy()
    bad[off[u]] = n_tok + 1
    bad[off[v] + 1] = -5
    groups.perm.copy_(torch.from_numpy(bad))
    out = torch.full_like(direct, float("nan"))
    lib().lookup(plan, d_ids, out=out, groups=groups)
    torch.cuda.synchronize()
    keep = np.ones(n_tok, bool)
    keep[lost] = False
    got, want = out.cpu().numpy(), direct.cpu().numpy()
    assert np.isnan(got[~keep]).all()
    assert np.array_equal(got[keep], want[keep])


def test_lookup_dedup_graph_replay_matches_eager():
    """dedup + fused dedup lookup captured into one HIP graph (no memset, no allocation); every replay on new ids
    gives the oracle's group count and the direct fused lookup's result bitwise."""
    _say("dedup + lookup dedup in a hip graph")
    plan = _small_plan(93, 4096)
    rng = np.random.default_rng(93)
    n_seq, seq_len, shared = 8, 300, 100

    def batch():
        prefix = rng.integers(0, 129280, size=shared).astype(np.int32)
        own = rng.integers(0, 129280, size=(n_seq, seq_len - shared)).astype(np.int32)
        return np.concatenate([np.tile(prefix, (n_seq, 1)), own], 1)

    ids = batch()
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = ids.size
    out = torch.empty((n_tok, 2, 256), dtype=torch.float32, device="cuda")
    groups = _new_groups(n_tok)
    ws = torch.empty(lib().dedup_workspace_bytes(plan, n_tok), dtype=torch.uint8, device="cuda")

    def step():
        lib().dedup(plan, d_ids, workspace=ws, groups=groups)
        lib().lookup(plan, d_ids, out=out, groups=groups)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the side stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        ids = batch()
        d_ids.copy_(torch.from_numpy(ids))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(groups.n_unique.item()) == oracle.dedup(oracle.windows(ids))[2], rep
        direct = lib().lookup(plan, d_ids)
        torch.cuda.synchronize()
        assert torch.equal(out, direct), rep
