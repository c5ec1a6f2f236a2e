"""Seeded synthetic workloads for the Engram lookup (inputs only).

This module generates the token ids and the FP8 tables that both the HIP path
and the CPU oracle consume.  It holds none of the lookup's arithmetic: no
windowing, no hashing, no decoding, no reduction.  The table contents are a
counter-based generator (``tablegen.c``) so that the full-size tables can be
produced on the device by a separate implementation of the same definition
and regenerated here, row by row, for any sampled token.

The five workloads follow the shapes the pages describe for this operator:

* 48 sub-tables per token (2 Engram modules x n-gram orders 2, 3, 4 x 8 hash
  heads), each row 256 FP8 bytes; the full tables hold ~196.6B parameters
  (2 x ~384M rows x 256), i.e. 2^24 rows per sub-table here.
  [How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup Table,
  sections "Where the 510 GB goes" and "Engram: the table that is never
  multiplied"]
* a 128K-token prefill as the headline case, decode of one new token per
  sequence against its history, and batched prompts that share a prefix
  [same page, "Engram: the table that is never multiplied"].

Token ids are Zipf(s=1.1) over a 129,280-entry vocabulary, drawn by inverse
CDF (numpy's own ``zipf`` is unbounded and is not used); the tiny case draws
uniform ids in [0, 1024).  No public benchmark or dataset is involved.
"""
from __future__ import annotations

import ctypes
import mmap
import os
import subprocess
from dataclasses import dataclass

import numpy as np

N_SUB = 48
ROW_BYTES = 256
VOCAB = 129_280
ZIPF_S = 1.1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tablegen.c")
_LIB = os.path.join(_HERE, "libtablegen.so")


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    ``ids`` are [n_seq, seq_len]; ``history`` (decode only) is [n_seq, 3] with
    history[s][2] the id just before position 0.  Positions before 0 with no
    history read as id 0.
    """

    key: int
    name: str
    n_seq: int
    seq_len: int
    rows: int
    ids_kind: str  # "uniform1024" | "zipf" | "zipf_shared_prefix"
    history: bool
    prefix_len: int = 0

    @property
    def n_tok(self) -> int:
        return self.n_seq * self.seq_len

    @property
    def table_seed(self) -> int:
        return 1000 + self.key

    @property
    def token_seed(self) -> int:
        return 2000 + self.key


WORKLOADS = {
    1: Workload(1, "tiny", 1, 512, 4096, "uniform1024", False),
    2: Workload(2, "decode", 64, 1, 1 << 20, "zipf", True),
    3: Workload(3, "prefill", 1, 32768, 1 << 22, "zipf", False),
    4: Workload(4, "full", 1, 131072, 1 << 24, "zipf", False),
    5: Workload(5, "batched_shared_prefix", 64, 8192, 1 << 24, "zipf_shared_prefix", False, 4096),
}


_ZIPF_CDF = None


def zipf_cdf(vocab: int = VOCAB, s: float = ZIPF_S) -> np.ndarray:
    global _ZIPF_CDF
    if vocab == VOCAB and s == ZIPF_S and _ZIPF_CDF is not None:
        return _ZIPF_CDF
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    if vocab == VOCAB and s == ZIPF_S:
        _ZIPF_CDF = cdf
    return cdf


def zipf_ids(rng: np.random.Generator, n: int, vocab: int = VOCAB, s: float = ZIPF_S) -> np.ndarray:
    """Ids = rank - 1 of a bounded Zipf(s) over ``vocab`` ranks, by inverse CDF."""
    u = rng.random(n)
    idx = np.searchsorted(zipf_cdf(vocab, s), u, side="right")
    return np.minimum(idx, vocab - 1).astype(np.int32)


def make_ids(w: Workload, token_seed: int | None = None):
    """Return (ids int32 [n_seq, seq_len], history int32 [n_seq, 3] or None)."""
    rng = np.random.Generator(np.random.PCG64(w.token_seed if token_seed is None else token_seed))
    if w.ids_kind == "uniform1024":
        ids = rng.integers(0, 1024, size=(w.n_seq, w.seq_len), dtype=np.int64).astype(np.int32)
        return ids, None
    if w.ids_kind == "zipf" and w.history:
        both = zipf_ids(rng, w.n_seq * (3 + w.seq_len)).reshape(w.n_seq, 3 + w.seq_len)
        return np.ascontiguousarray(both[:, 3:]), np.ascontiguousarray(both[:, :3])
    if w.ids_kind == "zipf":
        return zipf_ids(rng, w.n_tok).reshape(w.n_seq, w.seq_len), None
    if w.ids_kind == "zipf_shared_prefix":
        prefix = zipf_ids(rng, w.prefix_len)
        suffix = zipf_ids(rng, w.n_seq * (w.seq_len - w.prefix_len))
        suffix = suffix.reshape(w.n_seq, w.seq_len - w.prefix_len)
        ids = np.concatenate([np.broadcast_to(prefix, (w.n_seq, w.prefix_len)), suffix], axis=1)
        return np.ascontiguousarray(ids), None
    raise ValueError(w.ids_kind)


def uniform_ids(n_seq: int, seq_len: int, seed: int, vocab: int = VOCAB) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)


COMPRESSED_VOCAB = 99_092


def vocab_map(seed: int = 7, vocab: int = VOCAB, compressed: int = COMPRESSED_VOCAB) -> np.ndarray:
    """A seeded surjection of ``vocab`` raw ids onto ``compressed`` ids (uint32 [vocab]).

    Stands in for the normalisation table (case, accent and spacing folding
    into a 99,092-id vocabulary) that needs the real tokenizer: the first
    ``compressed`` ids map to a random permutation of the compressed range,
    every further id to a random compressed id, so many raw ids share one.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.empty(vocab, np.uint32)
    m[:compressed] = rng.permutation(compressed).astype(np.uint32)
    m[compressed:] = rng.integers(0, compressed, size=vocab - compressed).astype(np.uint32)
    return m


def prime_rows(count: int = N_SUB, below: int = 1 << 24) -> list[int]:
    """The ``count`` largest primes below ``below`` (a prime-sized bucket range per sub-table)."""
    def is_prime(n: int) -> bool:
        if n < 2 or n % 2 == 0:
            return n == 2
        f = 3
        while f * f <= n:
            if n % f == 0:
                return False
            f += 2
        return True
    out, n = [], below - 1
    while len(out) < count:
        if is_prime(n):
            out.append(n)
        n -= 1
    return out


# ---------------------------------------------------------------------------
# Table generator (host implementation of the counter-based definition)
# ---------------------------------------------------------------------------

_lib = None


def build_tablegen(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _tablegen():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_tablegen()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        lib.tablegen_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, p, ctypes.c_int64, p, p]
        lib.tablegen_scatter.argtypes = [ctypes.c_uint64, ctypes.c_uint32, p, ctypes.c_int64, p, p]
        lib.tablegen_range.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64, p, p]
        lib.tablegen_e8m0_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, p, ctypes.c_int64, p]
        lib.tablegen_e8m0_scatter.argtypes = [ctypes.c_uint64, ctypes.c_uint32, p, ctypes.c_int64, p]
        lib.tablegen_e8m0_range.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64, p]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def table_rows(seed: int, s: int, rows) -> tuple[np.ndarray, np.ndarray]:
    """Codes uint8 [n, 256] and scales float32 [n] of the given rows of sub-table s."""
    rows = np.ascontiguousarray(rows, dtype=np.uint32)
    codes = np.empty((rows.size, ROW_BYTES), np.uint8)
    scales = np.empty(rows.size, np.float32)
    _tablegen().tablegen_rows(seed, s, _ptr(rows), rows.size, _ptr(codes), _ptr(scales))
    return codes, scales


def table_range(seed: int, s: int, r0: int, n: int) -> tuple[np.ndarray, np.ndarray]:
    codes = np.empty((n, ROW_BYTES), np.uint8)
    scales = np.empty(n, np.float32)
    _tablegen().tablegen_range(seed, s, r0, n, _ptr(codes), _ptr(scales))
    return codes, scales


def e8m0_rows(seed: int, s: int, rows) -> np.ndarray:
    """E8M0 block scales uint8 [n, 8] of the given rows of sub-table s."""
    rows = np.ascontiguousarray(rows, dtype=np.uint32)
    out = np.empty((rows.size, 8), np.uint8)
    _tablegen().tablegen_e8m0_rows(seed, s, _ptr(rows), rows.size, _ptr(out))
    return out


def e8m0_range(seed: int, s: int, r0: int, n: int) -> np.ndarray:
    out = np.empty((n, 8), np.uint8)
    _tablegen().tablegen_e8m0_range(seed, s, r0, n, _ptr(out))
    return out


def dense_tables(seed: int, rows: int, scale_format: str = "f32_row") -> tuple[list, list]:
    """All 48 sub-tables in host memory (small row counts only).

    ``scale_format`` "f32_row": scales float32 [rows]; "e8m0_block32": uint8 [rows, 8].
    """
    tabs, scs = [], []
    for s in range(N_SUB):
        c, sc = table_range(seed, s, 0, rows)
        tabs.append(c)
        scs.append(sc if scale_format == "f32_row" else e8m0_range(seed, s, 0, rows))
    return tabs, scs


class SparseHostTables:
    """Full-size host tables of which only the needed rows are materialised.

    Each sub-table is a [rows, 256] uint8 view of one anonymous, lazily
    committed mapping, so its addressing is that of the real table while the
    resident memory is only the pages that hold requested rows.
    """

    def __init__(self, seed: int, rows: int, scale_format: str = "f32_row"):
        self.seed, self.rows, self.scale_format = seed, rows, scale_format
        nbytes = N_SUB * rows * ROW_BYTES
        flags = mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS | getattr(mmap, "MAP_NORESERVE", 0x4000)  # Linux value
        self._tab_map = mmap.mmap(-1, nbytes, flags=flags)
        self._sc_map = mmap.mmap(-1, N_SUB * rows * (4 if scale_format == "f32_row" else 8), flags=flags)
        tab = np.frombuffer(self._tab_map, dtype=np.uint8).reshape(N_SUB, rows, ROW_BYTES)
        if scale_format == "f32_row":
            sc = np.frombuffer(self._sc_map, dtype=np.float32).reshape(N_SUB, rows)
        else:
            sc = np.frombuffer(self._sc_map, dtype=np.uint8).reshape(N_SUB, rows, 8)
        self.tables = [tab[s] for s in range(N_SUB)]
        self.scales = [sc[s] for s in range(N_SUB)]

    def materialise(self, addr: np.ndarray) -> None:
        """Fill every row that ``addr`` ([n, 48] row indices) refers to."""
        addr = np.asarray(addr)
        for s in range(N_SUB):
            need = np.unique(addr[:, s]).astype(np.uint32)
            f32 = self.scale_format == "f32_row"
            _tablegen().tablegen_scatter(self.seed, s, _ptr(need), need.size,
                                         _ptr(self.tables[s]), _ptr(self.scales[s]) if f32 else None)
            if not f32:
                _tablegen().tablegen_e8m0_scatter(self.seed, s, _ptr(need), need.size, _ptr(self.scales[s]))

    def close(self) -> None:
        self.tables = self.scales = None
        for m in (self._tab_map, self._sc_map):
            try:
                m.close()
            except BufferError:
                pass
