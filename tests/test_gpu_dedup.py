"""GPU parity of the dedup pass: groups bit-exact against the oracle, and
dedup-mode memory vectors bitwise equal to direct mode."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import device_tables, dummy_plan, lib, small_device_tables, to_dev_ids

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_groups(groups, ids, hist):
    n_tok = ids.size
    want_perm, want_off, want_nu = oracle.dedup(oracle.windows(ids, hist))
    nu = int(groups.n_unique.item())
    assert nu == want_nu
    assert np.array_equal(groups.perm.cpu().numpy(), want_perm)
    assert np.array_equal(groups.offsets[:nu + 1].cpu().numpy(), want_off)
    assert want_off[-1] == n_tok


@pytest.mark.parametrize("n_seq,seq_len,hi,with_hist,vocab", [
    (1, 1, 10, False, 0), (1, 2, 1, False, 1), (1, 5, 3, True, 3), (2, 300, 4, False, 0), (3, 1000, 100, True, 100),
    (8, 517, 1 << 31, False, 0), (1, 5000, 2, False, 2), (64, 1, 129280, True, 129280),
    (4, 4096, 1 << 24, True, 1 << 24), (3, 3000, 129280, False, 129280), (2, 2500, 70000, True, 0),
])
def test_dedup_groups_exact(n_seq, seq_len, hi, with_hist, vocab):
    _say(f"dedup {n_seq}x{seq_len} ids<{hi} hist={with_hist} vocab={vocab}")
    rng = np.random.default_rng(seq_len + n_seq)
    ids = rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    hist = rng.integers(0, hi, size=(n_seq, 3), dtype=np.int64).astype(np.int32) if with_hist else None
    plan = dummy_plan(4096, vocab)
    groups = lib().dedup(plan, *to_dev_ids(ids, hist))
    torch.cuda.synchronize()
    _check_groups(groups, ids, hist)


_VOCABS = (0, 7, 1000, 65536, 65537, 129280, 1 << 18, (1 << 18) + 1, 1 << 20)


@pytest.mark.parametrize("case", range(24))
def test_dedup_random_shapes(case):
    """A seeded sweep over batch shapes, vocabulary sizes (both sides of the compacted-key range, and no bound),
    id ranges from a handful of values (long runs of equal windows, skewed digits) to the whole vocabulary, with and
    without history: groups exact against the oracle."""
    rng = np.random.default_rng(9000 + case)
    n_seq = int(rng.integers(1, 65))
    seq_len = int(rng.integers(1, max(2, 60000 // n_seq)))
    vocab = int(_VOCABS[case % len(_VOCABS)])
    top = vocab if vocab else 1 << 31
    hi = int(min(top, [3, 50, 5000, top][int(rng.integers(0, 4))]))
    with_hist = bool(rng.integers(0, 2))
    _say(f"dedup random case {case}: {n_seq}x{seq_len} ids<{hi} vocab={vocab} hist={with_hist}")
    ids = rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    hist = rng.integers(0, hi, size=(n_seq, 3), dtype=np.int64).astype(np.int32) if with_hist else None
    plan = dummy_plan(4096, vocab)
    groups = lib().dedup(plan, *to_dev_ids(ids, hist))
    torch.cuda.synchronize()
    _check_groups(groups, ids, hist)


def test_dedup_shared_prefix_batch():
    """Sequences sharing a prefix collapse to one group per prefix position."""
    _say("dedup shared prefix 16 x (256 + 256)")
    rng = np.random.default_rng(5)
    prefix = rng.integers(0, 129280, size=256).astype(np.int32)
    ids = np.concatenate([np.tile(prefix, (16, 1)), rng.integers(0, 129280, size=(16, 256)).astype(np.int32)], 1)
    plan = dummy_plan(4096, 129280)
    groups = lib().dedup(plan, *to_dev_ids(ids, None))
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)
    assert int(groups.n_unique.item()) <= 256 + 16 * 256


def test_dedup_empty():
    _say("dedup empty")
    plan = dummy_plan(4096)
    ids = torch.zeros((0, 5), dtype=torch.int32, device="cuda")
    groups = lib().dedup(plan, ids, None)
    torch.cuda.synchronize()
    assert int(groups.n_unique.item()) == 0 and int(groups.offsets[0].item()) == 0


def test_dedup_mode_equals_direct_small():
    _say("dedup-mode gather == direct (small)")
    R = 1024
    host_t, host_c = workloads.dense_tables(77, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, vocab_size=6)
    rng = np.random.default_rng(2)
    ids = rng.integers(0, 6, size=(7, 333)).astype(np.int32)  # many repeated windows
    d_ids, _ = to_dev_ids(ids, None)
    addr = lib().hash(plan, d_ids)
    direct = lib().gather_reduce(plan, addr)
    groups = lib().dedup(plan, d_ids)
    dd = torch.full_like(direct, float("nan"))
    lib().gather_reduce(plan, addr, out=dd, groups=groups)
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)
    assert torch.equal(dd, direct)


def test_dedup_pipeline_graph_replay_matches_eager():
    """hash + dedup + dedup-mode gather (about 30 launches, no memset or allocation) capture into one HIP graph;
    every replay on new ids gives the oracle's groups and the direct-mode result bitwise."""
    _say("dedup pipeline in a hip graph")
    R = 4096
    host_t, host_c = workloads.dense_tables(78, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, vocab_size=129280)
    rng = np.random.default_rng(9)
    n_seq, seq_len, shared = 8, 300, 100

    def batch():
        prefix = rng.integers(0, 129280, size=shared).astype(np.int32)
        own = rng.integers(0, 129280, size=(n_seq, seq_len - shared)).astype(np.int32)
        return np.concatenate([np.tile(prefix, (n_seq, 1)), own], 1)

    ids = batch()
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = ids.size
    addr = torch.empty((n_tok, 48), dtype=torch.uint32, device="cuda")
    out = torch.empty((n_tok, 2, 256), dtype=torch.float32, device="cuda")
    groups = lib().Groups(torch.empty(n_tok, dtype=torch.int32, device="cuda"),
                          torch.empty(n_tok + 1, dtype=torch.int32, device="cuda"),
                          torch.empty(1, dtype=torch.int32, device="cuda"))
    ws = torch.empty(lib().dedup_workspace_bytes(plan, n_tok), dtype=torch.uint8, device="cuda")

    def step():
        lib().hash(plan, d_ids, out=addr)
        lib().dedup(plan, d_ids, workspace=ws, groups=groups)
        lib().gather_reduce(plan, addr, out=out, groups=groups)

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
        _check_groups(groups, ids, None)
        direct = lib().gather_reduce(plan, lib().hash(plan, d_ids))
        torch.cuda.synchronize()
        assert torch.equal(out, direct), rep


def test_dedup_batched_shared_prefix_full_size():
    """The batched shared-prefix workload at full size: exact groups, dedup == direct bitwise."""
    w = workloads.WORKLOADS[5]
    _say(f"dedup workload 5 full size n_tok={w.n_tok}")
    ids, hist = workloads.make_ids(w)
    t, c = device_tables(w.rows, w.table_seed)
    plan = lib().Plan(t, c, vocab_size=workloads.VOCAB)
    d_ids, d_hist = to_dev_ids(ids, hist)
    addr = lib().hash(plan, d_ids, d_hist)
    direct = lib().gather_reduce(plan, addr)
    groups = lib().dedup(plan, d_ids, d_hist)
    dd = torch.full_like(direct, float("nan"))
    lib().gather_reduce(plan, addr, out=dd, groups=groups)
    torch.cuda.synchronize()
    _check_groups(groups, ids, hist)
    nu = int(groups.n_unique.item())
    _say(f"n_unique={nu} of {w.n_tok}")
    assert nu < w.n_tok * 0.6
    assert torch.equal(dd, direct)


def test_dedup_wide_keys_many_ids():
    """300,000 tokens uniform over a 129,280-id vocabulary use more than 2^16 distinct ids, so the compacted keys
    need 17 bits per id: 68-bit keys and a ninth pass over the high key word."""
    _say("dedup 3 x 100000 uniform ids, vocab 129280 (keys above 64 bits)")
    rng = np.random.default_rng(68)
    ids = rng.integers(0, 129280, size=(3, 100000), dtype=np.int64).astype(np.int32)
    plan = dummy_plan(4096, 129280)
    groups = lib().dedup(plan, *to_dev_ids(ids, None))
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)


def _ws_ids_in_use(ws):
    """The number of distinct ids the last compacting dedup call counted (a word of the workspace's control
    block, at byte 16)."""
    return int(ws[16:20].cpu().numpy().view(np.uint32)[0])


def test_dedup_workspace_state_across_calls():
    """The workspace is not cleared between calls: ids of an earlier call are not counted again, an arbitrary
    initial content is harmless, and a content that marks every id as in use still gives exact groups."""
    _say("dedup workspace reuse")
    plan = dummy_plan(4096, 129280)
    rng = np.random.default_rng(70)
    n_seq, seq_len = 4, 5000
    ws = torch.empty(lib().dedup_workspace_bytes(plan, n_seq * seq_len), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    for rep, hi in enumerate((129280, 500, 129280, 37)):
        ids = rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
        groups = lib().dedup(plan, *to_dev_ids(ids, None), workspace=ws)
        torch.cuda.synchronize()
        _check_groups(groups, ids, None)
        used = np.unique(np.concatenate([ids.ravel(), [0]])).size  # the ids plus the pad id 0
        if rep > 0:  # the first call may count stale entries of the 0xA5 fill
            assert _ws_ids_in_use(ws) == used, rep
    # every presence entry equal to the next call's stamp: all 129,280 ids count as in use (17-bit ids)
    words = ws.view(torch.int32)
    words.fill_(7)
    words[0] = 6  # the stamp of the "previous" call
    ids = rng.integers(0, 1000, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    groups = lib().dedup(plan, *to_dev_ids(ids, None), workspace=ws)
    torch.cuda.synchronize()
    assert _ws_ids_in_use(ws) == 129280
    _check_groups(groups, ids, None)


@pytest.mark.parametrize("vocab", [65536, 65537, 1 << 18, (1 << 18) + 1])
def test_dedup_vocab_bounds_of_compaction(vocab):
    """Vocabulary sizes at both edges of the compacted-key range give exact groups."""
    _say(f"dedup vocab {vocab}")
    rng = np.random.default_rng(vocab % 1000)
    ids = rng.integers(0, vocab, size=(5, 3001), dtype=np.int64).astype(np.int32)
    ids[:, :50] = vocab - 1 - np.arange(50)
    hist = rng.integers(0, vocab, size=(5, 3), dtype=np.int64).astype(np.int32)
    plan = dummy_plan(4096, vocab)
    groups = lib().dedup(plan, *to_dev_ids(ids, hist))
    torch.cuda.synchronize()
    _check_groups(groups, ids, hist)


def test_dedup_at_the_token_limit():
    """2^22 tokens, the most one call takes (1,024 tiles: every pass tile sums up to 1,023 earlier tiles' counts in
    8 rounds of 16 loads per thread column), ids uniform over a 129,280-id vocabulary (17-bit compacted keys)."""
    n_seq, seq_len = 4, 1 << 20
    _say(f"dedup {n_seq} x {seq_len} tokens (the per-call limit)")
    rng = np.random.default_rng(22)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    plan = dummy_plan(4096, 129280)
    groups = lib().dedup(plan, *to_dev_ids(ids, None))
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)


def test_dedup_gives_up_safely_when_a_wait_is_cut_short(monkeypatch):
    """With the wait bound forced to 0 polls (ENGRAM_DEDUP_SPIN_LIMIT), a tile that finds an earlier tile's counts
    not yet published gives up at once.  The call then reports n_unique = -1 and the dedup-mode gather writes
    nothing, or, if no tile had to wait, the result is exact; every kernel exits normally either way.  A call
    with the normal bound on the same workspace is exact again."""
    _say("dedup with the wait bound forced to 0")
    R = 1024
    host_t, host_c = workloads.dense_tables(79, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, vocab_size=129280)
    rng = np.random.default_rng(80)
    ids = rng.integers(0, 129280, size=(8, 40000)).astype(np.int32)  # 80 tiles per pass
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = ids.size
    ws = torch.empty(lib().dedup_workspace_bytes(plan, n_tok), dtype=torch.uint8, device="cuda")
    addr = lib().hash(plan, d_ids)
    direct = lib().gather_reduce(plan, addr)
    gave_up = 0
    for rep in range(3):
        monkeypatch.setenv("ENGRAM_DEDUP_SPIN_LIMIT", "0")
        groups = lib().dedup(plan, d_ids, workspace=ws)
        monkeypatch.delenv("ENGRAM_DEDUP_SPIN_LIMIT")
        out = torch.full_like(direct, float("nan"))
        lib().gather_reduce(plan, addr, out=out, groups=groups)
        torch.cuda.synchronize()
        nu = int(groups.n_unique.item())
        if nu == -1:
            gave_up += 1
            assert bool(torch.isnan(out).all())
        else:
            _check_groups(groups, ids, None)
            assert torch.equal(out, direct)
    _say(f"gave up in {gave_up} of 3 calls")
    groups = lib().dedup(plan, d_ids, workspace=ws)
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)


def _skewed_ids(pattern, rng, n_seq, seq_len):
    if pattern == "one-window":  # every window (0, 0, 0, 0): a single group of all tokens
        return np.zeros((n_seq, seq_len), dtype=np.int32)
    if pattern == "two-ids":  # 16 windows, each repeated ~32,000 times
        return rng.integers(0, 2, size=(n_seq, seq_len)).astype(np.int32)
    if pattern == "heavy-plus-spread":  # 60% of ids one value: one window holds ~13% of tokens, the rest spread
        ids = rng.integers(0, 129280, size=(n_seq, seq_len)).astype(np.int32)
        ids[rng.random((n_seq, seq_len)) < 0.6] = 5
        return ids
    if pattern == "periodic":  # every sequence repeats one 97-token pattern: 97 windows, ~5,400 tokens each
        base = rng.integers(0, 129280, size=97).astype(np.int32)
        return np.tile(base, (n_seq, seq_len // 97 + 1))[:, :seq_len]
    raise ValueError(pattern)


@pytest.mark.parametrize("pattern", ["one-window", "two-ids", "heavy-plus-spread", "periodic"])
def test_dedup_heavily_repeated_windows(pattern):
    """64 x 8,192 tokens whose windows repeat heavily (one window; 16 windows; one window holding ~13% of the
    tokens beside uniform ones; a 97-token period): a pass's digit is then one value for most of a tile, and
    groups run to hundreds of thousands of members.  Groups exact against the oracle."""
    n_seq, seq_len = 64, 8192
    _say(f"dedup repeated windows {pattern} {n_seq}x{seq_len}")
    rng = np.random.default_rng(len(pattern))
    ids = _skewed_ids(pattern, rng, n_seq, seq_len)
    plan = dummy_plan(4096, 129280)
    groups = lib().dedup(plan, *to_dev_ids(ids, None))
    torch.cuda.synchronize()
    _check_groups(groups, ids, None)
