"""Python binding of libengram.so, the Engram n-gram memory lookup for MI355X.

Argument marshalling only: every step of the lookup runs in the library's
HIP kernels.  PyTorch provides device memory and streams.  The library must
be built (``python hashed_gram_memory_amd/build.py``); importing this package
without it raises ImportError -- there is no fallback path.

Functions mirror the C ABI in include/engram.h:

    plan = Plan(tables, scales)                 # engram_plan
    addr = hash(plan, ids, history)             # engram_hash
    out  = gather_reduce(plan, addr)            # engram_gather_reduce
    groups = dedup(plan, ids, history)          # engram_dedup
    out  = gather_reduce(plan, addr, groups=groups)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loads the process's HIP runtime before the library binds to it

N_MODULES = 2
N_SUB = 48
ROW_BYTES = 256
N_MULT = 192
DEFAULT_HASH_SEED = 0x454E4752414D0001
SCALE_F32_ROW = 0
SCALE_E8M0_BLOCK32 = 1
_SCALE_FORMATS = {"f32_row": SCALE_F32_ROW, "e8m0_block32": SCALE_E8M0_BLOCK32}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")
MEASURE_LIB_PATH = os.path.join(_HERE, "libengram_measure.so")  # synthetic fill and ceiling probes (not the lookup)

STATUS = {0: "ENGRAM_OK", -1: "ENGRAM_EINVAL", -2: "ENGRAM_ERANGE", -3: "ENGRAM_EWORKSPACE",
          -4: "ENGRAM_EHIP", -5: "ENGRAM_EUNSUPPORTED"}


class EngramError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.engram_status_string(status).decode()} ({status})")


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("n_modules", ctypes.c_uint32),
        ("min_order", ctypes.c_uint32),
        ("max_order", ctypes.c_uint32),
        ("n_heads", ctypes.c_uint32),
        ("row_bytes", ctypes.c_uint32),
        ("vocab_size", ctypes.c_uint32),
        ("hash_seed", ctypes.c_uint64),
        ("rows", ctypes.POINTER(ctypes.c_uint64)),
        ("tables", ctypes.POINTER(ctypes.c_void_p)),
        ("scales", ctypes.POINTER(ctypes.c_void_p)),
        ("scale_format", ctypes.c_uint32),
        ("reserved1", ctypes.c_uint32),
        ("vocab_map", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python hashed_gram_memory_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, U64, U32, VP = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
    sig = {
        "engram_plan_desc_init": [ctypes.POINTER(PlanDesc)],
        "engram_plan": [ctypes.POINTER(PlanDesc), ctypes.POINTER(P)],
        "engram_plan_destroy": [P],
        "engram_plan_multipliers": [P, ctypes.POINTER(ctypes.c_uint64)],
        "engram_hash": [P, VP, VP, I64, I64, VP, VP],
        "engram_gather_reduce": [P, VP, I64, VP, VP, VP, VP, VP],
        "engram_lookup": [P, VP, VP, I64, I64, VP, VP],
        "engram_lookup_dedup": [P, VP, VP, I64, I64, VP, VP, VP, VP, VP],
        "engram_gather_reduce_batched": [P, VP, I64, I64, VP, VP],
        "engram_gather_weighted": [P, VP, I64, VP, VP, VP],
        "engram_gather_rows": [P, VP, I64, VP, VP],
        "engram_dedup_workspace": [P, I64, ctypes.POINTER(ctypes.c_size_t)],
        "engram_dedup": [P, VP, VP, I64, I64, VP, VP, VP, VP, ctypes.c_size_t, VP],
        "engram_dedup_noalloc": [P, VP, VP, I64, I64, VP, VP, VP, VP],
        "engram_check_inputs": [P, VP, VP, I64, I64, VP, I64, VP, VP],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.engram_status_string.argtypes = [ctypes.c_int]
    lib.engram_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()
_measure_lib = None


def lib() -> ctypes.CDLL:
    return _lib


def measure_lib() -> ctypes.CDLL:
    """libengram_measure.so: the seeded synthetic table fill and the memory-ceiling probes (loaded on first use)."""
    global _measure_lib
    if _measure_lib is None:
        if not os.path.exists(MEASURE_LIB_PATH):
            raise ImportError(f"{MEASURE_LIB_PATH} is not built; run `python hashed_gram_memory_amd/build.py`")
        m = ctypes.CDLL(MEASURE_LIB_PATH)
        P, I64, U64, U32, VP = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
        sig = {
            "engram_synth_fill": [VP, VP, U64, U32, U64, VP],
            "engram_synth_fill_e8m0": [VP, U64, U32, U64, VP],
            "engram_probe_read": [VP, U64, VP, VP],
            "engram_probe_copy": [VP, VP, U64, VP],
            "engram_probe_rows": [P, VP, I64, VP, VP],
            "engram_probe_random": [VP, U64, U32, U64, U64, VP, VP],
            "engram_probe_records": [VP, U64, U32, I64, U64, VP, VP],
        }
        for name, args in sig.items():
            fn = getattr(m, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _measure_lib = m
    return _measure_lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise EngramError(status, what)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream or None
    return int(stream) or None


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class Plan:
    """An immutable lookup plan over 48 device sub-tables.

    ``tables``: one uint8 tensor [48, R, 256] or a list of 48 tensors
    [R_s, 256]; ``scales``: float32 [48, R] / 48 x [R_s] ("f32_row"), or
    uint8 [48, R, 8] / 48 x [R_s, 8] ("e8m0_block32").  The tensors are
    referenced (not copied) and kept alive by the plan.
    """

    def __init__(self, tables, scales, hash_seed: int = DEFAULT_HASH_SEED, vocab_size: int = 0,
                 scale_format: str = "f32_row", vocab_map: torch.Tensor | None = None):
        if scale_format not in _SCALE_FORMATS:
            raise ValueError(f"scale_format must be one of {sorted(_SCALE_FORMATS)}")
        mx = scale_format == "e8m0_block32"
        if isinstance(tables, torch.Tensor):
            if tables.dim() != 3 or tables.shape[0] != N_SUB or tables.shape[2] != ROW_BYTES:
                raise ValueError("tables must be [48, R, 256]")
            tables = list(tables.unbind(0))
        if isinstance(scales, torch.Tensor):
            if scales.dim() != (3 if mx else 2) or scales.shape[0] != N_SUB:
                raise ValueError("scales must be [48, R, 8]" if mx else "scales must be [48, R]")
            scales = list(scales.unbind(0))
        if len(tables) != N_SUB or len(scales) != N_SUB:
            raise ValueError("need 48 tables and 48 scale vectors")
        rows = []
        for s in range(N_SUB):
            t, c = tables[s], scales[s]
            want = (t.shape[0], 8) if mx else (t.shape[0],)
            if t.dim() != 2 or t.shape[1] != ROW_BYTES or tuple(c.shape) != want:
                raise ValueError(f"sub-table {s}: need table [R, 256] and scales {list(want)}")
            _dev(t, torch.uint8, f"tables[{s}]")
            _dev(c, torch.uint8 if mx else torch.float32, f"scales[{s}]")
            rows.append(t.shape[0])
        map_ptr = None
        if vocab_map is not None:
            if vocab_map.dim() != 1:
                raise ValueError("vocab_map must be 1-D [vocab_size]")
            if vocab_size == 0:
                vocab_size = vocab_map.shape[0]
            if vocab_map.shape[0] != vocab_size:
                raise ValueError("vocab_map length must equal vocab_size")
            map_ptr = _dev(vocab_map, vocab_map.dtype if vocab_map.dtype in (torch.int32, torch.uint32)
                           else torch.int32, "vocab_map")
        self._build(rows, [t.data_ptr() for t in tables], [c.data_ptr() for c in scales], hash_seed, vocab_size,
                    keep=(tables, scales, vocab_map), scale_format=_SCALE_FORMATS[scale_format], vocab_map=map_ptr)

    @classmethod
    def from_pointers(cls, rows, table_ptrs, scale_ptrs, hash_seed: int = DEFAULT_HASH_SEED, vocab_size: int = 0,
                      keep=None, scale_format: str = "f32_row", vocab_map_ptr: int | None = None) -> "Plan":
        """Plan over raw device pointers (48 each) with the given row counts; ``keep`` is held alive."""
        p = cls.__new__(cls)
        p._build(list(rows), list(table_ptrs), list(scale_ptrs), hash_seed, vocab_size, keep,
                 scale_format=_SCALE_FORMATS[scale_format], vocab_map=vocab_map_ptr)
        return p

    def _build(self, rows, tab_ptrs, sc_ptrs, hash_seed, vocab_size, keep, scale_format: int = SCALE_F32_ROW,
               vocab_map: int | None = None) -> None:
        if len(rows) != N_SUB or len(tab_ptrs) != N_SUB or len(sc_ptrs) != N_SUB:
            raise ValueError("need 48 row counts, table pointers and scale pointers")
        self._handle = None
        self.rows = rows
        self.hash_seed = hash_seed
        self.vocab_size = vocab_size
        self.scale_format = scale_format
        self._keep = keep
        self._rows_c = (ctypes.c_uint64 * N_SUB)(*rows)
        self._tabs_c = (ctypes.c_void_p * N_SUB)(*tab_ptrs)
        self._scs_c = (ctypes.c_void_p * N_SUB)(*sc_ptrs)
        desc = PlanDesc()
        _check(_lib.engram_plan_desc_init(ctypes.byref(desc)), "engram_plan_desc_init")
        desc.hash_seed = hash_seed
        desc.vocab_size = vocab_size
        desc.scale_format = scale_format
        desc.vocab_map = vocab_map
        desc.rows = ctypes.cast(self._rows_c, ctypes.POINTER(ctypes.c_uint64))
        desc.tables = ctypes.cast(self._tabs_c, ctypes.POINTER(ctypes.c_void_p))
        desc.scales = ctypes.cast(self._scs_c, ctypes.POINTER(ctypes.c_void_p))
        handle = ctypes.c_void_p()
        _check(_lib.engram_plan(ctypes.byref(desc), ctypes.byref(handle)), "engram_plan")
        self._handle = handle

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._handle

    def multipliers(self) -> list[int]:
        buf = (ctypes.c_uint64 * N_MULT)()
        _check(_lib.engram_plan_multipliers(self._handle, buf), "engram_plan_multipliers")
        return list(buf)

    def close(self) -> None:
        if getattr(self, "_handle", None):
            _lib.engram_plan_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ids_shape(ids: torch.Tensor, history):
    if ids.dim() != 2:
        raise ValueError("ids must be [n_seq, seq_len]")
    n_seq, seq_len = ids.shape
    if history is not None and tuple(history.shape) != (n_seq, 3):
        raise ValueError("history must be [n_seq, 3]")
    return n_seq, seq_len


def hash(plan: Plan, ids: torch.Tensor, history: torch.Tensor | None = None, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """48 row addresses per token: uint32 [n_seq*seq_len, 48] (engram_hash)."""
    n_seq, seq_len = _ids_shape(ids, history)
    n_tok = n_seq * seq_len
    if out is None:
        out = torch.empty((n_tok, N_SUB), dtype=torch.uint32, device=ids.device)
    elif tuple(out.shape) != (n_tok, N_SUB):
        raise ValueError("out must be [n_tok, 48]")
    st = _lib.engram_hash(plan.handle, _dev(ids, torch.int32, "ids"),
                          None if history is None else _dev(history, torch.int32, "history"),
                          n_seq, seq_len, _dev(out, torch.uint32, "addr"), _stream(stream))
    _check(st, "engram_hash")
    return out


@dataclass
class Groups:
    """Result of dedup: device perm [n_tok], offsets [n_tok+1], n_unique [1]."""

    perm: torch.Tensor
    offsets: torch.Tensor
    n_unique: torch.Tensor


def _check_groups(groups: Groups, n_tok: int) -> None:
    """A Groups must be sized for exactly n_tok tokens: perm [n_tok], offsets [n_tok + 1], n_unique [>= 1]."""
    if not isinstance(groups, Groups):
        raise TypeError("groups must be a Groups")
    for name, t, want in (("perm", groups.perm, n_tok), ("offsets", groups.offsets, n_tok + 1)):
        if not isinstance(t, torch.Tensor) or t.dim() != 1 or t.shape[0] != want:
            raise ValueError(f"groups.{name} must be a 1-D tensor of {want} elements for {n_tok} tokens")
    if not isinstance(groups.n_unique, torch.Tensor) or groups.n_unique.numel() < 1:
        raise ValueError("groups.n_unique must hold at least one element")


def gather_reduce(plan: Plan, addr: torch.Tensor, out: torch.Tensor | None = None, groups: Groups | None = None,
                  stream=None) -> torch.Tensor:
    """Per-module sum of the 24 dequantised rows: fp32 [n_tok, 2, 256] (engram_gather_reduce)."""
    if addr.dim() != 2 or addr.shape[1] != N_SUB:
        raise ValueError("addr must be [n_tok, 48]")
    n_tok = addr.shape[0]
    if out is None:
        out = torch.empty((n_tok, N_MODULES, ROW_BYTES), dtype=torch.float32, device=addr.device)
    elif tuple(out.shape) != (n_tok, N_MODULES, ROW_BYTES):
        raise ValueError("out must be [n_tok, 2, 256]")
    perm = offsets = n_unique = None
    if groups is not None:
        _check_groups(groups, n_tok)
        perm = _dev(groups.perm, torch.int32, "perm")
        offsets = _dev(groups.offsets, torch.int32, "offsets")
        n_unique = _dev(groups.n_unique, torch.int32, "n_unique")
    st = _lib.engram_gather_reduce(plan.handle, _dev(addr, torch.uint32, "addr"), n_tok, perm, offsets, n_unique,
                                   _dev(out, torch.float32, "out"), _stream(stream))
    _check(st, "engram_gather_reduce")
    return out


def lookup(plan: Plan, ids: torch.Tensor, history: torch.Tensor | None = None, out: torch.Tensor | None = None,
           groups: Groups | None = None, stream=None) -> torch.Tensor:
    """Hash and gather-reduce in one launch: fp32 [n_seq*seq_len, 2, 256] (engram_lookup).  With ``groups`` from
    dedup() of the same ids: one hash and gather per group, the same result (engram_lookup_dedup)."""
    n_seq, seq_len = _ids_shape(ids, history)
    n_tok = n_seq * seq_len
    if out is None:
        out = torch.empty((n_tok, N_MODULES, ROW_BYTES), dtype=torch.float32, device=ids.device)
    elif tuple(out.shape) != (n_tok, N_MODULES, ROW_BYTES):
        raise ValueError("out must be [n_tok, 2, 256]")
    hist = None if history is None else _dev(history, torch.int32, "history")
    if groups is None:
        st = _lib.engram_lookup(plan.handle, _dev(ids, torch.int32, "ids"), hist, n_seq, seq_len,
                                _dev(out, torch.float32, "out"), _stream(stream))
        _check(st, "engram_lookup")
        return out
    _check_groups(groups, n_tok)
    st = _lib.engram_lookup_dedup(plan.handle, _dev(ids, torch.int32, "ids"), hist, n_seq, seq_len,
                                  _dev(groups.perm, torch.int32, "perm"), _dev(groups.offsets, torch.int32, "offsets"),
                                  _dev(groups.n_unique, torch.int32, "n_unique"), _dev(out, torch.float32, "out"),
                                  _stream(stream))
    _check(st, "engram_lookup_dedup")
    return out


def gather_reduce_batched(plan: Plan, addr: torch.Tensor, n_seq: int, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """engram_gather_reduce over a batch of ``n_seq`` equal-length sequences (addr [n_seq*seq_len, 48] in token order),
    visiting tokens in the batch order: fp32 [n_tok, 2, 256] (engram_gather_reduce_batched)."""
    if addr.dim() != 2 or addr.shape[1] != N_SUB:
        raise ValueError("addr must be [n_tok, 48]")
    n_tok = addr.shape[0]
    if n_seq <= 0 or n_tok % n_seq:
        raise ValueError("n_seq must divide the token count")
    if out is None:
        out = torch.empty((n_tok, N_MODULES, ROW_BYTES), dtype=torch.float32, device=addr.device)
    elif tuple(out.shape) != (n_tok, N_MODULES, ROW_BYTES):
        raise ValueError("out must be [n_tok, 2, 256]")
    st = _lib.engram_gather_reduce_batched(plan.handle, _dev(addr, torch.uint32, "addr"), n_seq, n_tok // n_seq,
                                           _dev(out, torch.float32, "out"), _stream(stream))
    _check(st, "engram_gather_reduce_batched")
    return out


def gather_weighted(plan: Plan, addr: torch.Tensor, weights: torch.Tensor, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Per-module sum with one caller weight per row: fp32 [n_tok, 2, 256] (engram_gather_weighted)."""
    if addr.dim() != 2 or addr.shape[1] != N_SUB or tuple(weights.shape) != tuple(addr.shape):
        raise ValueError("addr and weights must be [n_tok, 48]")
    n_tok = addr.shape[0]
    if out is None:
        out = torch.empty((n_tok, N_MODULES, ROW_BYTES), dtype=torch.float32, device=addr.device)
    elif tuple(out.shape) != (n_tok, N_MODULES, ROW_BYTES):
        raise ValueError("out must be [n_tok, 2, 256]")
    st = _lib.engram_gather_weighted(plan.handle, _dev(addr, torch.uint32, "addr"), n_tok,
                                     _dev(weights, torch.float32, "weights"), _dev(out, torch.float32, "out"),
                                     _stream(stream))
    _check(st, "engram_gather_weighted")
    return out


def gather_rows(plan: Plan, addr: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The 48 dequantised rows of every token: fp32 [n_tok, 48, 256] (engram_gather_rows)."""
    if addr.dim() != 2 or addr.shape[1] != N_SUB:
        raise ValueError("addr must be [n_tok, 48]")
    n_tok = addr.shape[0]
    if out is None:
        out = torch.empty((n_tok, N_SUB, ROW_BYTES), dtype=torch.float32, device=addr.device)
    elif tuple(out.shape) != (n_tok, N_SUB, ROW_BYTES):
        raise ValueError("out must be [n_tok, 48, 256]")
    st = _lib.engram_gather_rows(plan.handle, _dev(addr, torch.uint32, "addr"), n_tok, _dev(out, torch.float32, "rows"),
                                 _stream(stream))
    _check(st, "engram_gather_rows")
    return out


def dedup_workspace_bytes(plan: Plan, n_tok: int) -> int:
    """Workspace bytes of dedup for n_tok tokens under this plan (engram_dedup_workspace)."""
    b = ctypes.c_size_t()
    _check(_lib.engram_dedup_workspace(plan.handle, n_tok, ctypes.byref(b)), "engram_dedup_workspace")
    return b.value


def dedup(plan: Plan, ids: torch.Tensor, history: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          groups: Groups | None = None, stream=None) -> Groups:
    """Group tokens with equal id windows (engram_dedup)."""
    n_seq, seq_len = _ids_shape(ids, history)
    n_tok = n_seq * seq_len
    dev = ids.device
    if groups is None:
        groups = Groups(torch.empty(n_tok, dtype=torch.int32, device=dev),
                        torch.empty(n_tok + 1, dtype=torch.int32, device=dev),
                        torch.empty(1, dtype=torch.int32, device=dev))
    else:
        _check_groups(groups, n_tok)
    need = dedup_workspace_bytes(plan, n_tok)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = _lib.engram_dedup(plan.handle, _dev(ids, torch.int32, "ids"),
                           None if history is None else _dev(history, torch.int32, "history"), n_seq, seq_len,
                           _dev(groups.perm, torch.int32, "perm"), _dev(groups.offsets, torch.int32, "offsets"),
                           _dev(groups.n_unique, torch.int32, "n_unique"), _dev(workspace, torch.uint8, "workspace"),
                           workspace.numel(), _stream(stream))
    _check(st, "engram_dedup")
    return groups


def check_inputs(plan: Plan, ids: torch.Tensor | None = None, history: torch.Tensor | None = None,
                 addr: torch.Tensor | None = None, counts: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Count contract violations without faulting (engram_check_inputs): device int32 [3] = (negative ids, ids at or
    above the plan's vocab_size, addresses at or above their sub-table's row count)."""
    n_seq = seq_len = 0
    if ids is not None:
        n_seq, seq_len = _ids_shape(ids, history)
    elif history is not None:
        raise ValueError("history needs ids")
    n_addr = 0
    if addr is not None:
        if addr.dim() != 2 or addr.shape[1] != N_SUB:
            raise ValueError("addr must be [n_tok, 48]")
        n_addr = addr.shape[0]
    dev = (ids if ids is not None else addr).device if (ids is not None or addr is not None) else None
    if counts is None:
        if dev is None:
            raise ValueError("nothing to check")
        counts = torch.empty(3, dtype=torch.int32, device=dev)
    elif counts.numel() < 3:
        raise ValueError("counts must hold 3 int32")
    st = _lib.engram_check_inputs(plan.handle, None if ids is None else _dev(ids, torch.int32, "ids"),
                                  None if history is None else _dev(history, torch.int32, "history"), n_seq, seq_len,
                                  None if addr is None else _dev(addr, torch.uint32, "addr"), n_addr,
                                  _dev(counts, torch.int32, "counts"), _stream(stream))
    _check(st, "engram_check_inputs")
    return counts


DEDUP_SCRATCH_BYTES = 32 << 20


def dedup_noalloc(plan: Plan, ids: torch.Tensor, history: torch.Tensor | None = None, groups: Groups | None = None,
                  stream=None) -> Groups:
    """dedup with the library's fixed device workspace (engram_dedup_noalloc): the call allocates nothing when
    ``groups`` is given.  Calls that overlap on one GPU race."""
    n_seq, seq_len = _ids_shape(ids, history)
    n_tok = n_seq * seq_len
    if groups is None:
        groups = Groups(torch.empty(n_tok, dtype=torch.int32, device=ids.device),
                        torch.empty(n_tok + 1, dtype=torch.int32, device=ids.device),
                        torch.empty(1, dtype=torch.int32, device=ids.device))
    else:
        _check_groups(groups, n_tok)
    st = _lib.engram_dedup_noalloc(plan.handle, _dev(ids, torch.int32, "ids"),
                                   None if history is None else _dev(history, torch.int32, "history"), n_seq, seq_len,
                                   _dev(groups.perm, torch.int32, "perm"), _dev(groups.offsets, torch.int32, "offsets"),
                                   _dev(groups.n_unique, torch.int32, "n_unique"), _stream(stream))
    _check(st, "engram_dedup_noalloc")
    return groups


def synth_fill(tables, scales, seed: int, stream=None, scale_format: str = "f32_row") -> None:
    """Fill 48 sub-tables from the seeded generator (engram_synth_fill, engram_synth_fill_e8m0).

    ``tables``: uint8 [48, R, 256] or a list of 48 [R, 256]; ``scales``:
    float32 [48, R] / 48 x [R] ("f32_row") or uint8 [48, R, 8] / 48 x [R, 8]
    ("e8m0_block32").
    """
    mx = _SCALE_FORMATS[scale_format] == SCALE_E8M0_BLOCK32
    tables = list(tables.unbind(0)) if isinstance(tables, torch.Tensor) else list(tables)
    scales = list(scales.unbind(0)) if isinstance(scales, torch.Tensor) else list(scales)
    if len(tables) != N_SUB or len(scales) != N_SUB:
        raise ValueError("need 48 tables and 48 scale vectors")
    for s in range(N_SUB):
        t, c = tables[s], scales[s]
        want = (t.shape[0], 8) if mx else (t.shape[0],)
        if t.dim() != 2 or t.shape[1] != ROW_BYTES or tuple(c.shape) != want:
            raise ValueError(f"sub-table {s}: need table [R, 256] and scales {list(want)}")
        if mx:
            st = measure_lib().engram_synth_fill(_dev(t, torch.uint8, "table"), None, t.shape[0], s, seed, _stream(stream))
            _check(st, "engram_synth_fill")
            st = measure_lib().engram_synth_fill_e8m0(_dev(c, torch.uint8, "scales"), t.shape[0], s, seed, _stream(stream))
            _check(st, "engram_synth_fill_e8m0")
        else:
            st = measure_lib().engram_synth_fill(_dev(t, torch.uint8, "table"), _dev(c, torch.float32, "scales"), t.shape[0],
                                        s, seed, _stream(stream))
            _check(st, "engram_synth_fill")


# ---------------------------------------------------------------------------
# Memory-ceiling probes (measurement only; include/engram_probe.h)
# ---------------------------------------------------------------------------

def probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream-read every byte of the contiguous device tensor ``src``."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    _check(measure_lib().engram_probe_read(src.data_ptr(), nbytes - nbytes % 16, _dev(sink, torch.int32, "sink"),
                                  _stream(stream)), "engram_probe_read")


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Stream-copy ``src`` into ``dst`` (same byte size, contiguous, device)."""
    nbytes = src.numel() * src.element_size()
    if nbytes != dst.numel() * dst.element_size() or not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be device tensors of the same byte size")
    _check(measure_lib().engram_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes - nbytes % 16, _stream(stream)),
           "engram_probe_copy")


def probe_random(buf: torch.Tensor, chunk_bytes: int, read_bytes: int, sink: torch.Tensor, seed: int = 1,
                 stream=None) -> None:
    """Random reads of whole ``chunk_bytes`` chunks of the contiguous device tensor ``buf`` (engram_probe_random)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(measure_lib().engram_probe_random(buf.data_ptr(), buf.numel() * buf.element_size(), chunk_bytes, read_bytes, seed,
                                    _dev(sink, torch.int32, "sink"), _stream(stream)), "engram_probe_random")


PROBE_RECORD_LAYOUTS = ("rows_only", "separate_f32", "inline_f32_260", "inline_e8m0_264")


def probe_records(buf: torch.Tensor, layout: str, out: torch.Tensor, seed: int = 1, stream=None) -> None:
    """Random-row gather-sum with the row scales placed per ``layout`` (engram_probe_records); ``out`` is fp32
    [n_tok, 2, 256] and sets the token count."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if out.dtype != torch.float32 or out.dim() != 3 or tuple(out.shape[1:]) != (2, 256) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [n_tok, 2, 256] tensor")
    _check(measure_lib().engram_probe_records(buf.data_ptr(), buf.numel() * buf.element_size(),
                                     PROBE_RECORD_LAYOUTS.index(layout), out.shape[0], seed, out.data_ptr(),
                                     _stream(stream)), "engram_probe_records")


def probe_rows(plan: Plan, addr: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """The gather without its scale reads (engram_probe_rows)."""
    if addr.dim() != 2 or addr.shape[1] != N_SUB or tuple(out.shape) != (addr.shape[0], N_MODULES, ROW_BYTES):
        raise ValueError("addr must be [n_tok, 48] and out [n_tok, 2, 256]")
    _check(measure_lib().engram_probe_rows(plan.handle, _dev(addr, torch.uint32, "addr"), addr.shape[0],
                                  _dev(out, torch.float32, "out"), _stream(stream)), "engram_probe_rows")
    return out
