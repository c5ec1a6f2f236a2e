"""CPU oracle for the Engram n-gram memory read.

TEST INFRASTRUCTURE.  This module is the plain, slow, obviously correct
statement of what the lookup computes.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import or call it; the library path
never does.  It shares no code, tables or constants with the HIP library
beyond the seeded inputs both receive.

Sources (web pages; cited by title and section):

* [VRAM] "DeepSeek V4.1 Flash: The VRAM Killer. Can You Run It Locally?",
  section "What makes up the 511 GB of weights?"
* [GUIDE] "How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a
  Lookup Table", sections "The architecture" and "Engram: the table that is
  never multiplied"
* [REQ] "Running DeepSeek V4.1 Flash locally: the numbers beyond 552B",
  section "Backbone, Engram, and active parameters describe different scales"
* [X] "How DeepSeek V4.1 Flash's 763B weights run on consumer GPUs" (the
  repost names MXFP8 among the published Engram table widths)

What the pages fix: per token, suffix n-grams of order 2, 3 and 4 of the id
stream are hashed by 8 independent heads in each of two Engram modules, one
row is read per (order, head) pair, so 24 rows per module and 48 per token
[VRAM; GUIDE "Engram"]; the row indices depend on token ids alone [VRAM;
GUIDE "Engram"]; each row is 256 bytes of FP8 [GUIDE "Engram"; REQ].

What the pages leave open, and the reading taken here (each is listed in the
design notes):

* hash: per (module m, order n, head h) a multiply-xor of the window,
  x = XOR_{k<n} (u64(w_k) * M[m][n][h][k]) mod 2^64, row = x mod R_s;
  w_0 is the current token, w_k the id k positions back;
* multipliers: M[i] = (i+1)-th splitmix64 output seeded with the plan's hash
  seed, forced odd; i runs over (m, n, h, k) in that nesting, k over 0..3;
* sub-table order: s = 24*m + 8*(n-2) + h;
* positions before the sequence start take the caller's history ids, else 0;
* FP8 flavour: E4M3 in the OCP encoding (bias 7, one NaN pattern per sign,
  no infinities); one fp32 scale per row, or -- for the pages' 8 bytes of
  scales per row, read as the microscaling FP8 format the tables are named
  in [X] -- one E8M0 exponent per 32-element block;
* combination: the 24 dequantised rows of a module are summed.  The pages'
  learned gate needs trained weights and a hidden state and is not part of
  this operator.

Floating point here is float64.  For the synthetic tables (scales k * 2^-23
with k < 2^24) every product code*scale is a multiple of 2^-32 below 2^10 in
magnitude, so every partial sum of 24 of them is a multiple of 2^-32 below
2^15: float64 holds it exactly and the result does not depend on the
summation order.  The same holds for block scales 2^-7 .. 2^7 (products are
multiples of 2^-16 below 2^16).
"""
from __future__ import annotations

import math

import numpy as np

N_MODULES = 2
ORDERS = (2, 3, 4)
N_HEADS = 8
ROWS_PER_MODULE = len(ORDERS) * N_HEADS  # 24
N_SUB = N_MODULES * ROWS_PER_MODULE  # 48
ROW_BYTES = 256
WINDOW = max(ORDERS)  # 4
DEFAULT_HASH_SEED = 0x454E4752414D0001

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def sub_index(m: int, n: int, h: int) -> int:
    """Sub-table index of (module m, order n, head h): module-major, then order, then head."""
    return ROWS_PER_MODULE * m + N_HEADS * (n - ORDERS[0]) + h


# ---------------------------------------------------------------------------
# The id window of each token
# ---------------------------------------------------------------------------

def windows(ids, history=None, vocab_map=None) -> np.ndarray:
    """Window w[tok] = (w_0, w_1, w_2, w_3), w_k = id at position t - k.

    The suffix n-gram of order n ending at a token is (w_{n-1}, ..., w_0)
    [GUIDE "Engram"].  Positions before 0 read history[s][3 + (t - k)] when a
    history is given (history[s][2] is the id just before position 0), else 0.
    Tokens are numbered sequence-major: tok = s * seq_len + t.  With a
    ``vocab_map`` every window id is then normalised to vocab_map[id], the
    compressed vocabulary the pages' engines hash [GUIDE "Engram"].
    """
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim != 2:
        raise ValueError("ids must be [n_seq, seq_len]")
    n_seq, seq_len = ids.shape
    if history is None:
        pad = np.zeros((n_seq, WINDOW - 1), np.int64)
    else:
        pad = np.asarray(history, dtype=np.int64).reshape(n_seq, WINDOW - 1)
    ext = np.concatenate([pad, ids], axis=1)  # ext[s][3 + p] is the id at position p
    if np.any(ext < 0):
        raise ValueError("token ids must be non-negative")
    w = np.empty((n_seq, seq_len, WINDOW), np.int64)
    for k in range(WINDOW):
        w[:, :, k] = ext[:, WINDOW - 1 - k: WINDOW - 1 - k + seq_len]
    w = w.reshape(n_seq * seq_len, WINDOW)
    if vocab_map is not None:
        w = np.asarray(vocab_map, dtype=np.int64)[w]
    return w


# ---------------------------------------------------------------------------
# Hash: 48 addresses per token
# ---------------------------------------------------------------------------

def splitmix64(seed: int, count: int) -> list[int]:
    """First ``count`` outputs of splitmix64 (Steele, Lea and Flood 2014)."""
    state = seed & _MASK64
    out = []
    for _ in range(count):
        state = (state + _GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def multipliers(hash_seed: int = DEFAULT_HASH_SEED) -> np.ndarray:
    """Odd 64-bit multipliers M[m][n-2][h][k], uint64 [2, 3, 8, 4]."""
    vals = splitmix64(hash_seed, N_MODULES * len(ORDERS) * N_HEADS * WINDOW)
    return np.array([v | 1 for v in vals], dtype=np.uint64).reshape(
        N_MODULES, len(ORDERS), N_HEADS, WINDOW)


def hash_addresses(win: np.ndarray, mult: np.ndarray, rows) -> np.ndarray:
    """Row address of every (token, sub-table): uint32 [n_tok, 48].

    Eight heads per order and module, one row per (order, head) pair, each
    taken in its own bucket range of R_s rows [GUIDE "Engram"; VRAM].  The
    multiply-xor form and the modulus are this oracle's reading, which the
    library follows.
    """
    win = np.asarray(win, dtype=np.int64)
    rows = [int(r) for r in rows]
    if len(rows) != N_SUB or min(rows) < 1 or max(rows) > (1 << 32):
        raise ValueError("need 48 row counts in [1, 2^32]")
    w = win.astype(np.uint64)  # ids are non-negative int32: zero-extension
    addr = np.empty((win.shape[0], N_SUB), np.uint32)
    for m in range(N_MODULES):
        for n in ORDERS:
            for h in range(N_HEADS):
                x = np.zeros(win.shape[0], np.uint64)
                for k in range(n):  # the n most recent ids, w_0 .. w_{n-1}
                    x ^= w[:, k] * mult[m, n - ORDERS[0], h, k]  # wraps mod 2^64
                s = sub_index(m, n, h)
                addr[:, s] = x % np.uint64(rows[s])
    return addr


# ---------------------------------------------------------------------------
# FP8 E4M3 decode
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code: sign, 4-bit exponent (bias 7), 3-bit fraction.

    Exponent field 0 is subnormal (f * 2^-9); exponent 15 with fraction 7 is
    NaN; there is no infinity, so the largest finite magnitude is 448.
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        return sign * f * 2.0 ** -9
    return sign * (1.0 + f / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e8m0_value(e: int) -> float:
    """Value of an E8M0 scale byte: 2^(e - 127); the byte 255 is NaN (no sign, no mantissa)."""
    return math.nan if e == 255 else 2.0 ** (e - 127)


E8M0_TABLE = np.array([e8m0_value(e) for e in range(256)], dtype=np.float64)
SCALE_FORMATS = ("f32_row", "e8m0_block32")
BLOCK = 32  # elements per E8M0 scale


# ---------------------------------------------------------------------------
# Gather, dequantise, per-module sum
# ---------------------------------------------------------------------------

def row_scales(scales_s, a, scale_format: str) -> np.ndarray:
    """Scale of every element of the rows a of one sub-table: float64 [len(a), 256]."""
    if scale_format == "f32_row":
        sc = np.asarray(scales_s)[a].astype(np.float64)                 # one per row
        return np.repeat(sc[:, None], ROW_BYTES, axis=1)
    if scale_format == "e8m0_block32":
        e = np.asarray(scales_s)[a]                                     # [n, 8] bytes
        return np.repeat(E8M0_TABLE[e], BLOCK, axis=1)                  # element j uses byte j // 32
    raise ValueError(scale_format)


def gather_reduce(tables, scales, addr, scale_format: str = "f32_row") -> tuple[np.ndarray, np.ndarray]:
    """Memory vector of each token: float64 out [n_tok, 2, 256] and abs_sum.

    For module m and element j: out[tok][m][j] = sum over the module's 24
    sub-tables q of decode(T_{24m+q}[addr][j]) * scale_{24m+q}(addr, j)
    [GUIDE "Engram"; REQ], with one fp32 scale per row or one E8M0 scale per
    32-element block.  abs_sum is the same sum of absolute terms, the
    yardstick of the fp32 tolerance.
    """
    addr = np.asarray(addr)
    n_tok = addr.shape[0]
    out = np.zeros((n_tok, N_MODULES, ROW_BYTES), np.float64)
    abs_sum = np.zeros((n_tok, N_MODULES, ROW_BYTES), np.float64)
    for m in range(N_MODULES):
        for q in range(ROWS_PER_MODULE):
            s = ROWS_PER_MODULE * m + q
            a = addr[:, s].astype(np.int64)
            codes = np.asarray(tables[s])[a]                           # gather: [n_tok, 256] bytes
            sc = row_scales(scales[s], a, scale_format)                 # gather: [n_tok, 256]
            terms = E4M3_TABLE[codes] * sc                              # dequantise
            out[:, m, :] += terms                                       # per-module sum
            abs_sum[:, m, :] += np.abs(terms)
    return out, abs_sum


def gather_rows(tables, scales, addr, scale_format: str = "f32_row") -> np.ndarray:
    """The 48 dequantised rows of each token, un-reduced: float64 [n_tok, 48, 256].

    These are what the pages' learned gate weighs against the hidden state
    [GUIDE "The architecture", "Engram"].
    """
    addr = np.asarray(addr)
    rows = np.empty((addr.shape[0], N_SUB, ROW_BYTES), np.float64)
    for s in range(N_SUB):
        a = addr[:, s].astype(np.int64)
        rows[:, s, :] = E4M3_TABLE[np.asarray(tables[s])[a]] * row_scales(scales[s], a, scale_format)
    return rows


def gather_weighted(tables, scales, addr, weights, scale_format: str = "f32_row") -> tuple[np.ndarray, np.ndarray]:
    """Per-module sum with one weight per row: out[tok][m][j] = sum_q w[tok][24m+q] * row_{24m+q}[j].

    Returns (out, abs_sum) in float64, abs_sum being the sum of |terms|.
    """
    rows = gather_rows(tables, scales, addr, scale_format)
    terms = rows * np.asarray(weights, np.float64)[:, :, None]
    t = terms.reshape(terms.shape[0], N_MODULES, ROWS_PER_MODULE, ROW_BYTES)
    return t.sum(axis=2), np.abs(t).sum(axis=2)


def lookup(ids, history, tables, scales, rows, hash_seed: int = DEFAULT_HASH_SEED, scale_format: str = "f32_row",
           vocab_map=None):
    """Whole path: windows, hash, gather-reduce.  Returns (addr, out, abs_sum)."""
    addr = hash_addresses(windows(ids, history, vocab_map), multipliers(hash_seed), rows)
    out, abs_sum = gather_reduce(tables, scales, addr, scale_format)
    return addr, out, abs_sum


# ---------------------------------------------------------------------------
# Deduplication of equal windows
# ---------------------------------------------------------------------------

def dedup(win: np.ndarray) -> tuple[np.ndarray, np.ndarray, int]:
    """Group tokens with equal windows (w_0, w_1, w_2, w_3).

    Equal windows hash to equal addresses, so one lookup serves every token
    of a group.  Groups are ordered by ascending window (w_0 first, compared
    as unsigned), tokens within a group by ascending index.  Returns
    perm int32 [n_tok] (tokens group by group), offsets int32 [n_unique + 1]
    (offsets[u] = start of group u in perm, offsets[-1] = n_tok), n_unique.
    """
    win = np.asarray(win, dtype=np.int64)
    n_tok = win.shape[0]
    tok = np.arange(n_tok, dtype=np.int64)
    # np.lexsort sorts by the last key first: primary w_0, then w_1, w_2, w_3, then token index.
    perm = np.lexsort((tok, win[:, 3], win[:, 2], win[:, 1], win[:, 0]))
    sw = win[perm]
    first = np.ones(n_tok, dtype=bool)
    if n_tok > 1:
        first[1:] = np.any(sw[1:] != sw[:-1], axis=1)
    starts = np.flatnonzero(first)
    offsets = np.append(starts, n_tok).astype(np.int32)
    return perm.astype(np.int32), offsets, int(starts.size)
