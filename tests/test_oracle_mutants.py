"""Plant plausible mistakes in copies of the oracle; every one must fail a pin.

This shows the pins in pins.py are sharp enough: a dropped term, a wrong
sign, index, bias, order or operand anywhere in the oracle's steps is caught.
The mutants live here only; the oracle itself is never modified.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import engram_oracle as eo
import pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


# --------------------------------------------------------------------------- windows

def win_shift_by_one(ids, history=None):
    w = eo.windows(ids, history)
    n_seq, seq_len = np.asarray(ids).shape
    w = w.reshape(n_seq, seq_len, 4)
    out = np.zeros_like(w)
    out[:, :, 1:] = w[:, :, :3]
    out[:, :, 0] = w[:, :, 0]
    out[:, :, 1] = w[:, :, 0]  # w_1 duplicated from w_0
    return out.reshape(-1, 4)


def win_history_reversed(ids, history=None):
    if history is not None:
        history = np.asarray(history)[:, ::-1]
    return eo.windows(ids, history)


def win_reversed(ids, history=None):
    return eo.windows(ids, history)[:, ::-1]


def win_flattened_across_sequences(ids, history=None):
    ids = np.asarray(ids)
    w = eo.windows(ids.reshape(1, -1), None if history is None else np.asarray(history)[:1])
    return w


@pytest.mark.parametrize("mutant", [win_shift_by_one, win_history_reversed, win_reversed,
                                    win_flattened_across_sequences])
def test_window_mutants_caught(mutant):
    assert _fails(pins.check_windows, mutant)


# --------------------------------------------------------------------------- splitmix / multipliers

def splitmix_wrong_shift(seed, count):
    state, out, M = seed, [], (1 << 64) - 1
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & M
        z = state
        z = ((z ^ (z >> 31)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        out.append(z ^ (z >> 31))
    return out


def splitmix_off_by_one(seed, count):
    return eo.splitmix64(seed, count + 1)[1:]


@pytest.mark.parametrize("mutant", [splitmix_wrong_shift, splitmix_off_by_one])
def test_splitmix_mutants_caught(mutant):
    assert _fails(pins.check_splitmix, mutant)


def mult_not_odd(seed=eo.DEFAULT_HASH_SEED):
    vals = eo.splitmix64(seed, 192)
    return np.array(vals, dtype=np.uint64).reshape(2, 3, 8, 4)


def mult_shared_across_heads(seed=eo.DEFAULT_HASH_SEED):
    m = eo.multipliers(seed)
    return np.repeat(m[:, :, :1, :], 8, axis=2)


def mult_wrong_nesting(seed=eo.DEFAULT_HASH_SEED):
    m = eo.multipliers(seed)
    return np.ascontiguousarray(m.transpose(0, 1, 3, 2).reshape(2, 3, 4, 8).reshape(2, 3, 8, 4)[:, :, ::-1, :])


@pytest.mark.parametrize("mutant", [mult_not_odd, mult_shared_across_heads, mult_wrong_nesting])
def test_multiplier_mutants_caught(mutant):
    caught = _fails(pins.check_multipliers, mutant) or _fails(pins.check_hash, eo.hash_addresses, mutant)
    assert caught


# --------------------------------------------------------------------------- hash

def _hash_variant(term_range, combine, modulus, sub_fn=eo.sub_index):
    def h(win, mult, rows):
        win = np.asarray(win, np.int64)
        rows = [int(r) for r in rows]
        w = win.astype(np.uint64)
        addr = np.empty((win.shape[0], 48), np.uint32)
        for m in range(2):
            for n in (2, 3, 4):
                for hh in range(8):
                    x = np.zeros(win.shape[0], np.uint64)
                    for k in term_range(n):
                        x = combine(x, w[:, k] * mult[m, n - 2, hh, k])
                    s = sub_fn(m, n, hh)
                    addr[:, s] = modulus(x, rows[s])
        return addr
    return h


_xor = lambda x, t: x ^ t  # noqa: E731
_mod = lambda x, r: x % np.uint64(r)  # noqa: E731

HASH_MUTANTS = {
    "dropped_oldest_term": _hash_variant(lambda n: range(n - 1), _xor, _mod),
    "dropped_current_term": _hash_variant(lambda n: range(1, n), _xor, _mod),
    "one_term_too_many": _hash_variant(lambda n: range(min(n + 1, 4)), _xor, _mod),
    "add_instead_of_xor": _hash_variant(lambda n: range(n), lambda x, t: x + t, _mod),
    "mask_instead_of_mod": _hash_variant(lambda n: range(n), _xor,
                                         lambda x, r: (x & np.uint64(r - 1)) % np.uint64(r)),
    "high_bits": _hash_variant(lambda n: range(n), _xor, lambda x, r: (x >> np.uint64(32)) % np.uint64(r)),
    "order_head_swapped": _hash_variant(lambda n: range(n), _xor, _mod,
                                        sub_fn=lambda m, n, h: 24 * m + 3 * h + (n - 2)),
    "module_swapped": _hash_variant(lambda n: range(n), _xor, _mod,
                                    sub_fn=lambda m, n, h: 24 * (1 - m) + 8 * (n - 2) + h),
}


@pytest.mark.parametrize("name", sorted(HASH_MUTANTS))
def test_hash_mutants_caught(name):
    assert _fails(pins.check_hash, HASH_MUTANTS[name], eo.multipliers)


# --------------------------------------------------------------------------- decode

def _decode_table(fn):
    return np.array([fn(c) for c in range(256)], np.float64)


def dec_bias8(code):
    s = -1.0 if code & 0x80 else 1.0
    e, f = (code >> 3) & 15, code & 7
    if e == 15 and f == 7:
        return math.nan
    return s * (f * 2.0 ** -10 if e == 0 else (1 + f / 8) * 2.0 ** (e - 8))


def dec_no_subnormal(code):
    s = -1.0 if code & 0x80 else 1.0
    e, f = (code >> 3) & 15, code & 7
    if e == 15 and f == 7:
        return math.nan
    return s * (1 + f / 8) * 2.0 ** (e - 7)


def dec_unsigned(code):
    return abs(eo.e4m3_value(code))


def dec_fnuz(code):  # the other FP8 flavour: bias 8, NaN only at 0x80
    if code == 0x80:
        return math.nan
    s = -1.0 if code & 0x80 else 1.0
    e, f = (code >> 3) & 15, code & 7
    return s * (f * 2.0 ** -10 if e == 0 else (1 + f / 8) * 2.0 ** (e - 8))


def dec_inf_instead_of_nan(code):
    v = eo.e4m3_value(code)
    return math.copysign(math.inf, -1.0 if code & 0x80 else 1.0) if math.isnan(v) else v


@pytest.mark.parametrize("mutant", [dec_bias8, dec_no_subnormal, dec_unsigned, dec_fnuz, dec_inf_instead_of_nan])
def test_decode_mutants_caught(mutant):
    assert _fails(pins.check_decode, _decode_table(mutant))


# --------------------------------------------------------------------------- gather-reduce

def _gr_variant(sub_of=lambda m, q: 24 * m + q, q_range=range(24), row_of=lambda a, R: a,
                term=lambda d, sc: d * sc[:, None], table=None):
    dec = eo.E4M3_TABLE if table is None else table

    def gr(tables, scales, addr):
        addr = np.asarray(addr)
        n = addr.shape[0]
        out = np.zeros((n, 2, 256))
        ab = np.zeros((n, 2, 256))
        for m in range(2):
            for q in q_range:
                s = sub_of(m, q)
                R = np.asarray(tables[s]).shape[0]
                a = row_of(addr[:, s].astype(np.int64), R)
                t = term(dec[np.asarray(tables[s])[a]], np.asarray(scales[s])[a].astype(np.float64))
                out[:, m] += t
                ab[:, m] += np.abs(t)
        return out, ab
    return gr


GR_MUTANTS = {
    "module_swapped": _gr_variant(sub_of=lambda m, q: 24 * (1 - m) + q),
    "last_row_dropped": _gr_variant(q_range=range(23)),
    "first_row_dropped": _gr_variant(q_range=range(1, 24)),
    "neighbour_row": _gr_variant(row_of=lambda a, R: (a + 1) % R),
    "scale_ignored": _gr_variant(term=lambda d, sc: d),
    "scale_divides": _gr_variant(term=lambda d, sc: d / sc[:, None]),
    "scale_transposed": _gr_variant(term=lambda d, sc: d * sc[None, :1]),
    "sign_dropped": _gr_variant(table=np.abs(eo.E4M3_TABLE)),
    "modules_mixed": _gr_variant(sub_of=lambda m, q: 2 * q + m),
}


@pytest.mark.parametrize("name", sorted(GR_MUTANTS))
def test_gather_reduce_mutants_caught(name):
    assert _fails(pins.check_gather_reduce, GR_MUTANTS[name])


# --------------------------------------------------------------------------- dedup

def dd_unstable(win):
    perm, off, nu = eo.dedup(win)
    perm = perm.copy()
    for u in range(nu):
        perm[off[u]:off[u + 1]] = perm[off[u]:off[u + 1]][::-1]
    return perm, off, nu


def dd_descending(win):
    win = np.asarray(win, np.int64)
    perm, off, nu = eo.dedup(-win - 1)
    return perm, off, nu


def dd_three_ids(win):
    win = np.asarray(win, np.int64).copy()
    win[:, 3] = 0
    return eo.dedup(win)


def dd_last_id_first(win):
    win = np.asarray(win, np.int64)
    return eo.dedup(win[:, ::-1])


@pytest.mark.parametrize("mutant", [dd_unstable, dd_descending, dd_three_ids, dd_last_id_first])
def test_dedup_mutants_caught(mutant):
    assert _fails(pins.check_dedup, mutant)


def test_real_oracle_passes_every_pin():
    pins.check_windows(oracle.windows)
    pins.check_splitmix(oracle.splitmix64)
    pins.check_multipliers(oracle.multipliers)
    pins.check_decode(oracle.E4M3_TABLE)
    pins.check_dedup(oracle.dedup)


# --------------------------------------------------------------------------- E8M0 block scales

def _gr_e8m0_variant(block=32, bias=127, byte_of=lambda j, blk: j // blk):
    def gr(tables, scales, addr):
        addr = np.asarray(addr)
        n = addr.shape[0]
        out = np.zeros((n, 2, 256))
        ab = np.zeros((n, 2, 256))
        j = np.arange(256)
        for m in range(2):
            for q in range(24):
                s = 24 * m + q
                a = addr[:, s].astype(np.int64)
                e = np.asarray(scales[s])[a][:, np.minimum(byte_of(j, block), 7)].astype(np.float64)
                t = eo.E4M3_TABLE[np.asarray(tables[s])[a]] * 2.0 ** (e - bias)
                out[:, m] += t
                ab[:, m] += np.abs(t)
        return out, ab
    return gr


E8M0_MUTANTS = {
    "block_16": _gr_e8m0_variant(block=16),
    "block_64": _gr_e8m0_variant(block=64),
    "bias_128": _gr_e8m0_variant(bias=128),
    "bytes_reversed": _gr_e8m0_variant(byte_of=lambda j, blk: 7 - j // blk),
    "byte_by_lane_mod": _gr_e8m0_variant(byte_of=lambda j, blk: (j // 4) % 8),
}


@pytest.mark.parametrize("name", sorted(E8M0_MUTANTS))
def test_e8m0_mutants_caught(name):
    assert _fails(pins.check_gather_reduce_e8m0, E8M0_MUTANTS[name])


def test_e8m0_decode_mutants_caught():
    bias128 = np.array([math.nan if e == 255 else 2.0 ** (e - 128) for e in range(256)])
    no_nan = np.array([2.0 ** (e - 127) for e in range(256)])
    assert _fails(pins.check_e8m0, bias128)
    assert _fails(pins.check_e8m0, no_nan)


# --------------------------------------------------------------------------- gate inputs

def _rows_module_swapped(t, s, a, fmt="f32_row"):
    r = eo.gather_rows(t, s, a, fmt)
    return np.concatenate([r[:, 24:], r[:, :24]], axis=1)


def _weighted_transposed(t, s, a, w, fmt="f32_row"):
    w = np.asarray(w)
    return eo.gather_weighted(t, s, a, w[:, ::-1], fmt)


def _weighted_unweighted(t, s, a, w, fmt="f32_row"):
    return eo.gather_reduce(t, s, a, fmt)


@pytest.mark.parametrize("rows_fn,weighted_fn", [
    (_rows_module_swapped, eo.gather_weighted),
    (eo.gather_rows, _weighted_transposed),
    (eo.gather_rows, _weighted_unweighted),
])
def test_gate_input_mutants_caught(rows_fn, weighted_fn):
    assert _fails(pins.check_gate_inputs, rows_fn, weighted_fn, eo.gather_reduce)


def win_map_skips_pad(ids, history=None, vocab_map=None):
    w = eo.windows(ids, history)
    if vocab_map is None:
        return w
    mapped = np.asarray(vocab_map, np.int64)[w]
    n_seq, seq_len = np.asarray(ids).shape
    t = np.tile(np.arange(seq_len), n_seq)
    for k in range(4):
        pad = (t - k < 0) & (history is None)
        mapped[pad, k] = 0
    return mapped


def win_map_before_history(ids, history=None, vocab_map=None):
    if vocab_map is None:
        return eo.windows(ids, history)
    ids = np.asarray(vocab_map, np.int64)[np.asarray(ids)]
    return eo.windows(ids, history)


@pytest.mark.parametrize("mutant", [win_map_skips_pad, win_map_before_history])
def test_window_map_mutants_caught(mutant):
    assert _fails(pins.check_windows_map, mutant)
