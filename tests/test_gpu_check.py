"""engram_check_inputs: counts of planted out-of-range ids and addresses equal numpy's.  The planted values are only
ever given to the check, which reads nothing but the arrays themselves; no lookup kernel sees them."""
import numpy as np
import pytest
import torch

from gpu_support import dummy_plan, lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _expected(ids, hist, addr, vocab, rows):
    allids = np.concatenate([ids.ravel(), hist.ravel() if hist is not None else np.zeros(0, np.int64)]).astype(np.int64)
    neg = int((allids < 0).sum())
    big = int(((allids >= vocab) & (allids >= 0)).sum()) if vocab else 0
    bad = int((addr.astype(np.uint64) >= np.array(rows, dtype=np.uint64)[None, :]).sum()) if addr is not None else 0
    return [neg, big, bad]


@pytest.mark.parametrize("n_seq,seq_len,vocab,with_hist", [(1, 1, 5, True), (7, 3001, 129280, True),
                                                           (3, 100000, 0, False), (64, 1, 99092, True)])
def test_check_counts_planted_values(n_seq, seq_len, vocab, with_hist):
    _say(f"check {n_seq}x{seq_len} vocab={vocab} hist={with_hist}")
    rng = np.random.default_rng(n_seq + seq_len)
    rows = [int(r) for r in rng.integers(1, 1 << 20, size=48)]
    rows[5], rows[40] = 1, 1 << 32
    plan = lib().Plan.from_pointers(rows, [0x7F0000000000] * 48, [0x7F0000000000] * 48, vocab_size=vocab)
    hi = vocab if vocab else 1 << 31
    ids = rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64)
    n_bad = max(1, ids.size // 97)
    pos = rng.choice(ids.size, size=min(n_bad, ids.size), replace=False)
    ids.ravel()[pos] = rng.integers(-(1 << 31), 1 << 31, size=pos.size)  # negative and too-large ids
    ids = ids.astype(np.int32)
    hist = None
    if with_hist:
        hist = rng.integers(0, hi, size=(n_seq, 3), dtype=np.int64)
        hist[0, 1] = -3
        if vocab:
            hist[-1, 2] = vocab
        hist = hist.astype(np.int32)
    n_tok = ids.size
    addr = (rng.integers(0, 1 << 32, size=(n_tok, 48), dtype=np.uint64) % np.array(rows, dtype=np.uint64)).astype(np.uint32)
    bad = rng.choice(n_tok * 48, size=min(500, n_tok * 48), replace=False)
    addr.ravel()[bad] = rng.integers(0, 1 << 32, size=bad.size, dtype=np.uint64).astype(np.uint32)
    d_ids = torch.from_numpy(ids).cuda()
    d_hist = None if hist is None else torch.from_numpy(hist).cuda()
    d_addr = torch.from_numpy(addr.view(np.int32)).cuda().view(torch.uint32)
    counts = lib().check_inputs(plan, d_ids, d_hist, d_addr)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == _expected(ids, hist, addr, vocab, rows)
    # in-range inputs count nothing; ids alone and addresses alone
    ok_ids = torch.from_numpy(rng.integers(0, hi, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)).cuda()
    assert lib().check_inputs(plan, ok_ids).cpu().tolist() == [0, 0, 0]
    good = (rng.integers(0, 1 << 32, size=(n_tok, 48), dtype=np.uint64) % np.array(rows, dtype=np.uint64)).astype(np.uint32)
    good_d = torch.from_numpy(good.view(np.int32)).cuda().view(torch.uint32)
    assert lib().check_inputs(plan, addr=good_d).cpu().tolist() == [0, 0, 0]


def test_check_hashed_addresses_are_in_range():
    """The hash's own output is always in range, for any row counts."""
    rng = np.random.default_rng(11)
    rows = [int(r) for r in rng.integers(1, 1 << 32, size=48)]
    plan = dummy_plan(4096)
    plan = lib().Plan.from_pointers(rows, [plan._keep[0].data_ptr()] * 48, [plan._keep[1].data_ptr()] * 48,
                                    keep=plan._keep)
    ids = torch.from_numpy(rng.integers(0, 129280, size=(5, 20011)).astype(np.int32)).cuda()
    addr = lib().hash(plan, ids)
    assert lib().check_inputs(plan, ids, addr=addr).cpu().tolist() == [0, 0, 0]
