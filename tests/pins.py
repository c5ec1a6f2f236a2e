"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` takes the oracle function(s) under test as arguments and
raises AssertionError on the first violated fact, so the same checks run
against the real oracle (test_oracle_pins.py) and against oracles with a
planted mistake (test_oracle_mutants.py), which must each fail one of them.

What the checks rest on:
* published known-answer values of splitmix64 (the generator's literature);
* PyTorch's own float8_e4m3fn conversion (an independent OCP E4M3 decoder)
  and the format's textbook values;
* closed forms and algebraic facts of the hash: an odd multiplier is a
  bijection modulo 2^k, an order-n n-gram reads exactly n ids, R = 1 maps
  everything to row 0, arbitrary-precision integer evaluation;
* special tables whose memory vector is known in closed form (all zero,
  constant, one non-zero sub-table, address-revealing) and a dense one-hot
  matrix-product formulation of the gather-sum (numpy matmul);
* the defining properties of a sort-and-group, and Python's own sort;
* hand-worked windows for small id sequences.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

N_SUB = 48
RPM = 24
MASK64 = (1 << 64) - 1

# splitmix64 known-answer values: the first five outputs for seed 1234567,
# and the first output for seed 0, as published with the generator's
# reference implementation and reproduced across its ports.
SPLITMIX_KAT_1234567 = [
    6457827717110365317,
    3203168211198807973,
    9817491932198370423,
    4593380528125082431,
    16408922859458223821,
]
SPLITMIX_KAT_0_FIRST = 0xE220A8397B1DCDAF


def sub(m, n, h):
    return RPM * m + 8 * (n - 2) + h


# ---------------------------------------------------------------------------
# windows
# ---------------------------------------------------------------------------

def check_windows(windows_fn):
    w = windows_fn(np.array([[5, 6, 7, 8]], np.int32), None)
    assert np.array_equal(w, [[5, 0, 0, 0], [6, 5, 0, 0], [7, 6, 5, 0], [8, 7, 6, 5]]), w
    w = windows_fn(np.array([[5, 6, 7, 8]], np.int32), np.array([[1, 2, 3]], np.int32))
    assert np.array_equal(w, [[5, 3, 2, 1], [6, 5, 3, 2], [7, 6, 5, 3], [8, 7, 6, 5]]), w
    # sequences do not see each other; tokens are numbered sequence-major
    w = windows_fn(np.array([[5, 6], [7, 8]], np.int32), None)
    assert np.array_equal(w, [[5, 0, 0, 0], [6, 5, 0, 0], [7, 0, 0, 0], [8, 7, 0, 0]]), w
    w = windows_fn(np.array([[9], [4]], np.int32), np.array([[1, 2, 3], [10, 11, 12]], np.int32))
    assert np.array_equal(w, [[9, 3, 2, 1], [4, 12, 11, 10]]), w


# ---------------------------------------------------------------------------
# hash
# ---------------------------------------------------------------------------

def check_splitmix(splitmix_fn):
    assert splitmix_fn(1234567, 5) == SPLITMIX_KAT_1234567
    assert splitmix_fn(0, 1)[0] == SPLITMIX_KAT_0_FIRST


def check_multipliers(mult_fn):
    m = mult_fn(1234567)
    assert m.shape == (2, 3, 8, 4) and m.dtype == np.uint64
    flat = [int(v) for v in m.ravel()]
    assert all(v & 1 for v in flat), "multipliers must be odd"
    assert len(set(flat)) == len(flat), "multipliers must be distinct"
    assert flat[:5] == [v | 1 for v in SPLITMIX_KAT_1234567]


def _rand_windows(rng, n, hi=1 << 17):
    return rng.integers(0, hi, size=(n, 4), dtype=np.int64)


def check_hash(hash_fn, mult_fn):
    rng = np.random.default_rng(7)
    mult = mult_fn(0x454E4752414D0001)

    # R = 1: every address is row 0
    win = _rand_windows(rng, 64)
    assert not hash_fn(win, mult, [1] * N_SUB).any()

    # 48 in-range addresses per token for awkward row counts
    rows = [1 << 32, (1 << 32) - 1, 1000003, 4096, 3, 2] * 8
    addr = hash_fn(win, mult, rows)
    assert addr.shape == (64, N_SUB) and addr.dtype == np.uint32
    assert all(int(addr[:, s].max()) < rows[s] for s in range(N_SUB))

    # arbitrary-precision evaluation on a few windows
    for t in range(8):
        for m in range(2):
            for n in (2, 3, 4):
                for h in range(8):
                    x = 0
                    for k in range(n):
                        x ^= (int(win[t, k]) * int(mult[m, n - 2, h, k])) & MASK64
                    s = sub(m, n, h)
                    assert int(addr[t, s]) == x % rows[s], (t, s)

    # an odd multiplier is a bijection modulo 2^k: sweeping w_0 (or the
    # oldest id of the n-gram) over [0, R) must hit every row exactly once
    R = 4096
    base = _rand_windows(rng, 1)[0]
    for pos in (0, 1, 2, 3):
        sweep = np.tile(base, (R, 1))
        sweep[:, pos] = np.arange(R)
        addr = hash_fn(sweep, mult, [R] * N_SUB)
        for m in range(2):
            for n in (2, 3, 4):
                for h in range(8):
                    col = addr[:, sub(m, n, h)]
                    if pos < n:
                        assert np.unique(col).size == R, (pos, m, n, h)
                    else:  # an order-n n-gram does not read w_pos
                        assert np.unique(col).size == 1, (pos, m, n, h)

    # equal windows give equal rows, wherever they sit
    win = _rand_windows(rng, 200, hi=8)
    addr = hash_fn(win, mult, [1 << 20] * N_SUB)
    key = {}
    for t in range(200):
        k = tuple(win[t])
        if k in key:
            assert np.array_equal(addr[t], addr[key[k]])
        key[k] = t

    # heads, orders and modules are independent: two sub-tables agree on a
    # row only at the chance rate 1/R
    win = _rand_windows(rng, 4000)
    R = 1 << 16
    addr = hash_fn(win, mult, [R] * N_SUB).astype(np.int64)
    for a, b in itertools.combinations(range(N_SUB), 2):
        assert np.mean(addr[:, a] == addr[:, b]) < 0.01, (a, b)

    # rows are spread evenly (chi-square, 61 buckets, 244 expected per bucket)
    R = 61
    win = _rand_windows(rng, 61 * 244)
    addr = hash_fn(win, mult, [R] * N_SUB)
    for s in range(N_SUB):
        cnt = np.bincount(addr[:, s], minlength=R)
        chi2 = float(((cnt - 244.0) ** 2 / 244.0).sum())
        assert chi2 < 140.0, (s, chi2)  # 60 dof: p < 1e-7 above 140


# ---------------------------------------------------------------------------
# FP8 E4M3 decode
# ---------------------------------------------------------------------------

def check_decode(table):
    import torch

    table = np.asarray(table, dtype=np.float64)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert np.array_equal(table[~nan], ref[~nan])
    assert np.array_equal(np.signbit(table[~nan]), np.signbit(ref[~nan]))
    assert table[0x38] == 1.0 and table[0xB8] == -1.0
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert table[0x08] == 2.0 ** -6 and table[0x01] == 2.0 ** -9 and table[0x07] == 7 * 2.0 ** -9
    assert table[0x00] == 0.0 and not np.signbit(table[0x00])
    assert table[0x80] == 0.0 and np.signbit(table[0x80])
    assert math.isnan(table[0x7F]) and math.isnan(table[0xFF])
    assert np.isnan(table).sum() == 2 and not np.isinf(table).any()


# ---------------------------------------------------------------------------
# gather + dequantise + per-module sum
# ---------------------------------------------------------------------------

def _decode_ref():
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return ref.to(torch.float64).numpy()


def check_gather_reduce(gr_fn):
    rng = np.random.default_rng(11)
    R, N = 16, 40
    addr = rng.integers(0, R, size=(N, N_SUB)).astype(np.uint32)
    dec = _decode_ref()

    def rand_codes(shape):
        c = rng.integers(0, 254, size=shape)
        return np.where(c < 127, c, c + 1).astype(np.uint8)

    # all-zero tables give exactly zero
    tabs = [np.zeros((R, 256), np.uint8) for _ in range(N_SUB)]
    scs = [rng.uniform(0.5, 2.0, R).astype(np.float32) for _ in range(N_SUB)]
    out, ab = gr_fn(tabs, scs, addr)
    assert out.shape == (N, 2, 256) and not out.any() and not ab.any()

    # constant code c with scale 1: every element is 24 * decode(c)
    for c in (0x38, 0x7E, 0xB0, 0x01):
        tabs = [np.full((R, 256), c, np.uint8) for _ in range(N_SUB)]
        ones = [np.ones(R, np.float32) for _ in range(N_SUB)]
        out, ab = gr_fn(tabs, ones, addr)
        assert np.all(out == 24.0 * dec[c]) and np.all(ab == 24.0 * abs(dec[c])), hex(c)

    # one non-zero sub-table s: its module holds decode(row) * scale, the other is zero
    for s in (0, 5, 23, 24, 30, 47):
        tabs = [np.zeros((R, 256), np.uint8) for _ in range(N_SUB)]
        tabs[s] = rand_codes((R, 256))
        out, _ = gr_fn(tabs, scs, addr)
        m = s // RPM
        want = dec[tabs[s][addr[:, s].astype(np.int64)]] * scs[s][addr[:, s].astype(np.int64)][:, None].astype(np.float64)
        assert np.array_equal(out[:, m, :], want), s
        assert not out[:, 1 - m, :].any(), s

    # address-revealing tables: element q of module m equals the row read from sub-table 24m+q
    R2 = 1 << 12
    addr2 = rng.integers(0, R2, size=(N, N_SUB)).astype(np.uint32)
    tabs = []
    for s in range(N_SUB):
        t = np.zeros((R2, 256), np.uint8)
        t[:, s % RPM] = 0x38
        tabs.append(t)
    rscs = [np.arange(R2, dtype=np.float32) for _ in range(N_SUB)]
    out, _ = gr_fn(tabs, rscs, addr2)
    for m in range(2):
        assert np.array_equal(out[:, m, :RPM], addr2[:, RPM * m:RPM * (m + 1)].astype(np.float64))
        assert not out[:, m, RPM:].any()

    # dense formulation: out[:, m] = sum_q onehot(addr_q) @ (decode(T_q) * scale_q)
    tabs = [rand_codes((R, 256)) for _ in range(N_SUB)]
    out, ab = gr_fn(tabs, scs, addr)
    for m in range(2):
        want = np.zeros((N, 256))
        want_abs = np.zeros((N, 256))
        for q in range(RPM):
            s = RPM * m + q
            onehot = np.zeros((N, R))
            onehot[np.arange(N), addr[:, s].astype(np.int64)] = 1.0
            vals = dec[tabs[s]] * scs[s].astype(np.float64)[:, None]
            want += np.matmul(onehot, vals)
            want_abs += np.matmul(onehot, np.abs(vals))
        assert np.allclose(out[:, m], want, rtol=0, atol=1e-9 * np.abs(want_abs).max())
        assert np.allclose(ab[:, m], want_abs, rtol=1e-12, atol=0)

    # doubling every scale doubles the result exactly; token order commutes
    out2, _ = gr_fn(tabs, [2 * s for s in scs], addr)
    assert np.array_equal(out2, 2 * out)
    p = rng.permutation(N)
    outp, _ = gr_fn(tabs, scs, addr[p])
    assert np.array_equal(outp, out[p])


# ---------------------------------------------------------------------------
# dedup
# ---------------------------------------------------------------------------

def check_dedup_result(win, perm, offsets, n_unique):
    """The defining properties of the grouping (complete: they fix it uniquely)."""
    win = np.asarray(win, dtype=np.int64)
    n = win.shape[0]
    perm = np.asarray(perm, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    assert perm.shape == (n,) and np.array_equal(np.sort(perm), np.arange(n))
    assert offsets.shape == (n_unique + 1,) and offsets[0] == 0 and offsets[-1] == n
    assert np.all(np.diff(offsets) > 0)
    assert n_unique == len({tuple(r) for r in win.tolist()})
    prev = None
    for u in range(n_unique):
        members = perm[offsets[u]:offsets[u + 1]]
        keys = win[members]
        assert np.all(keys == keys[0]), u
        assert np.all(np.diff(members) > 0), u  # ascending token index within a group
        k = tuple(keys[0].tolist())
        if prev is not None:
            assert prev < k, u  # ascending window, w_0 most significant
        prev = k


def check_dedup(dedup_fn):
    rng = np.random.default_rng(3)
    for n, hi in ((0, 4), (1, 4), (7, 2), (300, 3), (500, 1000)):
        win = rng.integers(0, hi, size=(n, 4), dtype=np.int64)
        perm, offsets, nu = dedup_fn(win)
        check_dedup_result(win, perm, offsets, nu)
        # Python's own sort on (window, token) gives the same order
        order = sorted(range(n), key=lambda t: (tuple(win[t].tolist()), t))
        assert list(np.asarray(perm).tolist()) == order
        groups = [len(list(g)) for _, g in itertools.groupby(order, key=lambda t: tuple(win[t].tolist()))]
        assert list(np.diff(offsets).tolist()) == groups
    # ids above 2^31 - 1 never occur (int32 ids), but the order is unsigned on the full id range
    win = np.array([[5, 0, 0, 0], [1 << 30, 0, 0, 0], [5, 0, 0, 1], [0, 9, 9, 9]], np.int64)
    perm, offsets, nu = dedup_fn(win)
    assert list(np.asarray(perm).tolist()) == [3, 0, 2, 1] and nu == 4


# ---------------------------------------------------------------------------
# E8M0 block scales
# ---------------------------------------------------------------------------

def check_e8m0(table):
    """E8M0 decode against PyTorch's own float8_e8m0fnu conversion and the format's definition."""
    import torch

    table = np.asarray(table, dtype=np.float64)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(table[ok], ref[ok])
    assert table[127] == 1.0 and table[128] == 2.0 and table[126] == 0.5 and table[0] == 2.0 ** -127
    assert np.isnan(table[255]) and np.isnan(table).sum() == 1


def check_gather_reduce_e8m0(gr_fn):
    """Block scales: closed forms that fix which byte scales which element."""
    rng = np.random.default_rng(13)
    R, N = 8, 30
    addr = rng.integers(0, R, size=(N, N_SUB)).astype(np.uint32)
    dec = _decode_ref()
    # code 1.0 everywhere; byte b of every row = 127 + b - 3  -> element j = 24 * 2^(j//32 - 3)
    tabs = [np.full((R, 256), 0x38, np.uint8) for _ in range(N_SUB)]
    scs = [np.tile((124 + np.arange(8)).astype(np.uint8), (R, 1)) for _ in range(N_SUB)]
    out, ab = gr_fn(tabs, scs, addr)
    want = 24.0 * 2.0 ** (np.arange(256) // 32 - 3)
    assert np.array_equal(out, np.broadcast_to(want, out.shape)) and np.array_equal(ab, out)
    # one non-zero sub-table, random codes and exponents: element j = decode(code_j) * 2^(e[j//32]-127)
    for s in (0, 13, 30, 47):
        tabs = [np.zeros((R, 256), np.uint8) for _ in range(N_SUB)]
        c = rng.integers(0, 254, size=(R, 256))
        tabs[s] = np.where(c < 127, c, c + 1).astype(np.uint8)
        scs = [rng.integers(110, 140, size=(R, 8)).astype(np.uint8) for _ in range(N_SUB)]
        out, _ = gr_fn(tabs, scs, addr)
        a = addr[:, s].astype(np.int64)
        scale = 2.0 ** (scs[s][a].astype(np.float64) - 127)
        want = dec[tabs[s][a]] * np.repeat(scale, 32, axis=1)
        m = s // RPM
        assert np.array_equal(out[:, m], want), s
        assert not out[:, 1 - m].any()
    # row index: a row's own exponents, not a neighbour's
    tabs = [np.full((R, 256), 0x38, np.uint8) for _ in range(N_SUB)]
    scs = [np.repeat((120 + np.arange(R)).astype(np.uint8)[:, None], 8, axis=1) for _ in range(N_SUB)]
    out, _ = gr_fn(tabs, scs, addr)
    for m in range(2):
        want = sum(2.0 ** (120 + addr[:, RPM * m + q].astype(np.float64) - 127) for q in range(RPM))
        assert np.array_equal(out[:, m, 0], want)


# ---------------------------------------------------------------------------
# gate inputs: un-reduced rows and caller-weighted sums
# ---------------------------------------------------------------------------

def check_gate_inputs(rows_fn, weighted_fn, gr_fn):
    """Un-reduced rows and weighted sums against the plain sum and closed forms."""
    rng = np.random.default_rng(17)
    R, N = 32, 20
    addr = rng.integers(0, R, size=(N, N_SUB)).astype(np.uint32)
    c = rng.integers(0, 254, size=(N_SUB, R, 256))
    tabs = [np.where(x < 127, x, x + 1).astype(np.uint8) for x in c]
    scs = [(rng.integers(1 << 22, 1 << 24, size=R) * 2.0 ** -23).astype(np.float32) for _ in range(N_SUB)]
    dec = _decode_ref()
    rows = rows_fn(tabs, scs, addr)
    assert rows.shape == (N, N_SUB, 256)
    for s in (0, 11, 24, 47):  # each row is its own decode times its own scale
        a = addr[:, s].astype(np.int64)
        assert np.array_equal(rows[:, s], dec[tabs[s][a]] * scs[s][a].astype(np.float64)[:, None]), s
    out, _ = gr_fn(tabs, scs, addr)
    ones, _ = weighted_fn(tabs, scs, addr, np.ones((N, N_SUB)))
    assert np.array_equal(ones, out)  # unit weights: the plain sum
    assert np.array_equal(rows.reshape(N, 2, 24, 256).sum(axis=2), out)
    w = np.zeros((N, N_SUB))
    w[:, 5] = 1.0
    w[:, 40] = -2.0
    one, _ = weighted_fn(tabs, scs, addr, w)
    assert np.array_equal(one[:, 0], rows[:, 5]) and np.array_equal(one[:, 1], -2.0 * rows[:, 40])
    w = rng.uniform(-1, 1, size=(N, N_SUB))
    got, ab = weighted_fn(tabs, scs, addr, w)
    want = np.einsum("nsj,ns->nsj", rows, w).reshape(N, 2, 24, 256).sum(axis=2)
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
    assert np.all(ab >= np.abs(got) - 1e-9)


def check_windows_map(windows_fn):
    """Every window id -- history and the pad id 0 included -- goes through the map."""
    vmap = np.arange(20, dtype=np.uint32) + 100
    vmap[5] = vmap[6] = 9
    vmap[0] = 7
    w = windows_fn(np.array([[5, 6, 1]], np.int32), None, vmap)
    assert np.array_equal(w, [[9, 7, 7, 7], [9, 9, 7, 7], [101, 9, 9, 7]]), w
    w = windows_fn(np.array([[5]], np.int32), np.array([[2, 3, 6]], np.int32), vmap)
    assert np.array_equal(w, [[9, 9, 103, 102]]), w
    ident = np.arange(20, dtype=np.uint32)
    ids = np.random.default_rng(0).integers(0, 20, size=(3, 9)).astype(np.int32)
    assert np.array_equal(windows_fn(ids, None, ident), windows_fn(ids, None, None))
