"""Helpers shared by the GPU parity tests (device tables, oracle on samples)."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import workloads

FULL_ROWS = 1 << 24


def lib():
    import hashed_gram_memory_amd as hg
    return hg


@functools.lru_cache(maxsize=1)
def big_buffer():
    """One [48, 2^24, 256] code buffer and [48, 2^24] scales (195 GiB), shared by all tests.

    Smaller tables are views of its leading rows, one contiguous [R, 256]
    block per sub-table.
    """
    tabs = torch.empty((48, FULL_ROWS, 256), dtype=torch.uint8, device="cuda")
    scs = torch.empty((48, FULL_ROWS), dtype=torch.float32, device="cuda")
    return tabs, scs


@functools.lru_cache(maxsize=1)
def big_e8m0_buffer():
    """[48, 2^24, 8] E8M0 block scales (6 GiB), shared by the block-scale tests."""
    return torch.empty((48, FULL_ROWS, 8), dtype=torch.uint8, device="cuda")


_filled = {"key": None}


def device_tables(rows: int, seed: int, scale_format: str = "f32_row"):
    """48 device sub-tables of ``rows`` rows filled from the seeded generator (lists of views)."""
    tabs, scs = big_buffer()
    if scale_format == "e8m0_block32":
        scs = big_e8m0_buffer()
    t = [tabs[s, :rows] for s in range(48)]
    c = [scs[s, :rows] for s in range(48)]
    if _filled["key"] != (rows, seed, scale_format):
        lib().synth_fill(t, c, seed, scale_format=scale_format)
        torch.cuda.synchronize()
        _filled["key"] = (rows, seed, scale_format)
    return t, c


def mark_buffer_dirty():
    _filled["key"] = None


def small_device_tables(host_tabs, host_scs):
    t = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in host_tabs]
    c = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in host_scs]
    return t, c


def dummy_plan(rows: int, vocab_size: int = 0):
    """A plan whose tables are never read (hash and dedup tests): every pointer is one small buffer."""
    t = torch.zeros((1, 256), dtype=torch.uint8, device="cuda")
    c = torch.zeros(1, dtype=torch.float32, device="cuda")
    return lib().Plan.from_pointers([rows] * 48, [t.data_ptr()] * 48, [c.data_ptr()] * 48, vocab_size=vocab_size,
                                    keep=(t, c))


def to_dev_ids(ids, history):
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    d_hist = None if history is None else torch.from_numpy(np.ascontiguousarray(history, dtype=np.int32)).cuda()
    return d_ids, d_hist


def addr_to_host(addr: torch.Tensor) -> np.ndarray:
    return addr.view(torch.int32).cpu().numpy().view(np.uint32)


def sample_tokens(n_tok: int, k: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = set(int(t) for t in must if 0 <= t < n_tok)
    pick.update(range(min(4, n_tok)))
    pick.add(n_tok - 1)
    if n_tok > k:
        while len(pick) < k:
            pick.update(rng.choice(n_tok, size=k - len(pick), replace=False).tolist())
    else:
        pick.update(range(n_tok))
    return np.array(sorted(pick), dtype=np.int64)


def oracle_sampled(ids, history, rows: int, seed: int, tokens: np.ndarray, scale_format: str = "f32_row"):
    """Oracle addresses for all tokens and memory vectors for ``tokens`` (regenerated rows)."""
    addr = oracle.hash_addresses(oracle.windows(ids, history), oracle.multipliers(), [rows] * 48)
    sub = addr[tokens]
    host = workloads.SparseHostTables(seed, rows, scale_format)
    try:
        host.materialise(sub)
        out, abs_sum = oracle.gather_reduce(host.tables, host.scales, sub, scale_format)
    finally:
        host.close()
    return addr, out, abs_sum


def assert_within_tolerance(gpu: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, rel: float = 1e-5):
    """|gpu - ref| <= rel * sum|terms| per element; exact where the bound is 0; NaN where ref is NaN."""
    gpu = gpu.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(gpu), nan), "NaN positions differ"
    ok = ~nan
    err = np.abs(gpu[ok] - ref[ok])
    bound = rel * abs_sum[ok]
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{bad.sum()} elements out of tolerance; first: err={err[i]} bound={bound[i]}")


def batch_sample(n_seq: int, seq_len: int, k: int, seed: int, seqs=(0, 1), positions=()) -> np.ndarray:
    """``k`` token indices of an n_seq x seq_len batch (token = seq * seq_len + position), always including, for
    every sequence in ``seqs``, positions 0-3, 63-65, the given ``positions`` and the last position, plus the
    batch's first and last tokens; the rest uniform at random."""
    must = []
    for s in seqs:
        if not 0 <= s < n_seq:
            continue
        for p in (0, 1, 2, 3, 63, 64, 65, seq_len - 1, *positions):
            if 0 <= p < seq_len:
                must.append(s * seq_len + p)
    return sample_tokens(n_seq * seq_len, k, seed, must=must)


def unwritten_tokens(out: torch.Tensor) -> int:
    """Tokens of a NaN-initialised [n_tok, 2, 256] output whose first element of either module is still NaN."""
    return int(torch.isnan(out[:, :, 0]).any(dim=1).sum().item())
