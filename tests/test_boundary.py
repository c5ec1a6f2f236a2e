"""The C ABI on the host: exported symbols, validation, plans (no device work)."""
import ctypes
import glob
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, ERANGE, EWORKSPACE, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced: validation fails or no launch happens


@pytest.fixture(scope="module")
def hg():
    import hashed_gram_memory_amd as hg
    return hg


@pytest.fixture(scope="module")
def L(hg):
    return hg.lib()


def _declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_\w+)\s*\(", text)))


def test_every_header_is_covered():
    assert sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h"))) == [
        "engram.h", "engram_probe.h", "engram_synth.h"]


def test_every_declared_symbol_is_exported(hg, L):
    """engram.h is the lookup library's; engram_synth.h and engram_probe.h are the measurement library's, and the
    lookup library exports none of their symbols."""
    import ctypes as _ct
    lookup = _declared_functions("engram.h")
    measure = _declared_functions("engram_synth.h") + _declared_functions("engram_probe.h")
    assert len(lookup) >= 15 and len(measure) >= 7
    M = hg.measure_lib()
    for n in lookup:
        assert hasattr(L, n), n
    for n in measure:
        assert hasattr(M, n), n
    plain = _ct.CDLL(hg.LIB_PATH)
    for n in measure:
        assert not hasattr(plain, n), n


def _desc(hg, rows=None, tabs=None, scs=None):
    d = hg.PlanDesc()
    assert hg.lib().engram_plan_desc_init(ctypes.byref(d)) == OK
    rows = rows if rows is not None else [4096] * 48
    tabs = tabs if tabs is not None else [FAKE + 256 * s for s in range(48)]
    scs = scs if scs is not None else [FAKE + 4 * s for s in range(48)]
    keep = ((ctypes.c_uint64 * 48)(*rows), (ctypes.c_void_p * 48)(*tabs), (ctypes.c_void_p * 48)(*scs))
    d.rows = ctypes.cast(keep[0], ctypes.POINTER(ctypes.c_uint64))
    d.tables = ctypes.cast(keep[1], ctypes.POINTER(ctypes.c_void_p))
    d.scales = ctypes.cast(keep[2], ctypes.POINTER(ctypes.c_void_p))
    return d, keep


def _plan(hg, d):
    h = ctypes.c_void_p()
    st = hg.lib().engram_plan(ctypes.byref(d), ctypes.byref(h))
    return st, h


def test_desc_init_defaults(hg):
    d, _ = _desc(hg)
    assert (d.n_modules, d.min_order, d.max_order, d.n_heads, d.row_bytes) == (2, 2, 4, 8, 256)
    assert d.hash_seed == oracle.DEFAULT_HASH_SEED
    assert hg.lib().engram_plan_desc_init(None) == EINVAL


def test_plan_validation(hg):
    L = hg.lib()
    d, keep = _desc(hg)
    st, h = _plan(hg, d)
    assert st == OK and h.value
    assert L.engram_plan_destroy(h) == OK
    assert L.engram_plan_destroy(None) == OK
    assert L.engram_plan(None, ctypes.byref(ctypes.c_void_p())) == EINVAL
    assert L.engram_plan(ctypes.byref(d), None) == EINVAL
    for field, val in (("n_modules", 1), ("min_order", 1), ("max_order", 5), ("n_heads", 4), ("row_bytes", 128)):
        d2, k2 = _desc(hg)
        setattr(d2, field, val)
        assert _plan(hg, d2)[0] == EUNSUPPORTED, field
    for vocab in (1, 129280, (1 << 31), (1 << 32) - 1):
        d2, k2 = _desc(hg)
        d2.vocab_size = vocab
        st, h = _plan(hg, d2)
        assert st == OK
        L.engram_plan_destroy(h)
    for rows, want in (([0] * 48, ERANGE), ([(1 << 32) + 1] * 48, ERANGE), ([1 << 32] * 48, OK), ([1] * 48, OK)):
        d2, k2 = _desc(hg, rows=rows)
        st, h = _plan(hg, d2)
        assert st == want, rows[0]
        if st == OK:
            L.engram_plan_destroy(h)
    tabs = [FAKE] * 48
    tabs[7] = FAKE + 8  # not 16-byte aligned
    assert _plan(hg, _desc(hg, tabs=tabs)[0])[0] == EINVAL
    tabs[7] = 0
    assert _plan(hg, _desc(hg, tabs=tabs)[0])[0] == EINVAL
    scs = [FAKE] * 48
    scs[3] = FAKE + 2
    assert _plan(hg, _desc(hg, scs=scs)[0])[0] == EINVAL
    d2, k2 = _desc(hg)
    d2.rows = None
    assert _plan(hg, d2)[0] == EINVAL


def test_plan_multipliers_match_oracle(hg):
    """The library's host-side splitmix64 derivation agrees with the oracle's (independent code)."""
    for seed in (oracle.DEFAULT_HASH_SEED, 0, 1234567, (1 << 64) - 1):
        d, keep = _desc(hg)
        d.hash_seed = seed
        st, h = _plan(hg, d)
        assert st == OK
        buf = (ctypes.c_uint64 * 192)()
        assert hg.lib().engram_plan_multipliers(h, buf) == OK
        assert list(buf) == [int(v) for v in oracle.multipliers(seed).ravel()]
        hg.lib().engram_plan_destroy(h)


@pytest.fixture()
def plan(hg):
    d, keep = _desc(hg)
    st, h = _plan(hg, d)
    assert st == OK
    yield h
    hg.lib().engram_plan_destroy(h)


def test_hash_validation(hg, plan):
    L = hg.lib()
    assert L.engram_hash(None, FAKE, None, 1, 1, FAKE, None) == EINVAL
    assert L.engram_hash(plan, FAKE, None, 0, 100, FAKE, None) == OK  # no tokens: no launch
    assert L.engram_hash(plan, None, None, 0, 0, None, None) == OK
    assert L.engram_hash(plan, FAKE, None, -1, 4, FAKE, None) == EINVAL
    assert L.engram_hash(plan, FAKE, None, 4, -1, FAKE, None) == EINVAL
    assert L.engram_hash(plan, FAKE, None, 1 << 16, 1 << 15, FAKE, None) == ERANGE  # 2^31 tokens
    assert L.engram_hash(plan, None, None, 1, 1, FAKE, None) == EINVAL
    assert L.engram_hash(plan, FAKE, None, 1, 1, None, None) == EINVAL
    assert L.engram_hash(plan, FAKE + 2, None, 1, 1, FAKE, None) == EINVAL
    assert L.engram_hash(plan, FAKE, None, 1, 1, FAKE + 4, None) == EINVAL
    assert L.engram_hash(plan, FAKE, FAKE + 1, 1, 1, FAKE, None) == EINVAL


def test_gather_reduce_validation(hg, plan):
    L = hg.lib()
    assert L.engram_gather_reduce(None, FAKE, 1, None, None, None, FAKE, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 0, None, None, None, FAKE, None) == OK
    assert L.engram_gather_reduce(plan, FAKE, -1, None, None, None, FAKE, None) == ERANGE
    assert L.engram_gather_reduce(plan, FAKE, 1 << 31, None, None, None, FAKE, None) == ERANGE
    assert L.engram_gather_reduce(plan, None, 1, None, None, None, FAKE, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 1, None, None, None, None, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE + 4, 1, None, None, None, FAKE, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 1, None, None, None, FAKE + 8, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 1, FAKE, None, None, FAKE, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 1, FAKE, FAKE, None, FAKE, None) == EINVAL
    assert L.engram_gather_reduce(plan, FAKE, 1, FAKE + 1, FAKE, FAKE, FAKE, None) == EINVAL


def test_dedup_validation(hg, plan):
    L = hg.lib()
    b = ctypes.c_size_t()
    assert L.engram_dedup_workspace(plan, -1, ctypes.byref(b)) == ERANGE
    assert L.engram_dedup_workspace(plan, (1 << 22) + 1, ctypes.byref(b)) == ERANGE
    assert L.engram_dedup_workspace(plan, 1 << 22, ctypes.byref(b)) == OK
    assert L.engram_dedup_workspace(plan, 1, None) == EINVAL
    assert L.engram_dedup_workspace(None, 1, ctypes.byref(b)) == EINVAL
    assert L.engram_dedup_workspace(plan, 0, ctypes.byref(b)) == OK and b.value == 0
    assert L.engram_dedup_workspace(plan, 1000, ctypes.byref(b)) == OK
    need = b.value
    assert need > 0
    if need:
        assert L.engram_dedup(plan, FAKE, None, 1, 1000, FAKE, FAKE, FAKE, None, need, None) == EWORKSPACE
        assert L.engram_dedup(plan, FAKE, None, 1, 1000, FAKE, FAKE, FAKE, FAKE, need - 1, None) == EWORKSPACE
        assert L.engram_dedup(plan, FAKE, None, 1, 1000, FAKE, FAKE, FAKE, FAKE + 64, need, None) == EWORKSPACE
    assert L.engram_dedup(plan, FAKE, None, 1, 1000, None, FAKE, FAKE, FAKE, need, None) == EINVAL
    assert L.engram_dedup(plan, FAKE, None, 1, 1000, FAKE, None, FAKE, FAKE, need, None) == EINVAL
    assert L.engram_dedup(plan, FAKE, None, 1, 1000, FAKE, FAKE, None, FAKE, need, None) == EINVAL
    assert L.engram_dedup(plan, FAKE, None, -1, 1000, FAKE, FAKE, FAKE, FAKE, need, None) == EINVAL
    assert L.engram_dedup(None, FAKE, None, 1, 1000, FAKE, FAKE, FAKE, FAKE, need, None) == EINVAL
    assert L.engram_dedup(plan, FAKE, None, 1 << 11, (1 << 11) + 1, FAKE, FAKE, FAKE, FAKE, need, None) == ERANGE


def test_synth_fill_validation(hg):
    M = hg.measure_lib()
    L = hg.lib()
    assert M.engram_synth_fill(FAKE, FAKE, 0, 0, 1, None) == ERANGE
    assert M.engram_synth_fill(FAKE, FAKE, (1 << 32) + 1, 0, 1, None) == ERANGE
    assert M.engram_synth_fill(FAKE, FAKE, 16, 48, 1, None) == EINVAL
    assert M.engram_synth_fill(FAKE + 4, FAKE, 16, 0, 1, None) == EINVAL
    assert M.engram_synth_fill(FAKE, FAKE + 2, 16, 0, 1, None) == EINVAL


def test_status_strings(hg):
    L = hg.lib()
    for st in (OK, EINVAL, ERANGE, EWORKSPACE, EHIP, EUNSUPPORTED):
        assert L.engram_status_string(st).decode().startswith(hg.STATUS[st])
    assert b"unknown" in L.engram_status_string(-99)


def test_binding_rejects_host_tensors(hg):
    import torch
    with pytest.raises(ValueError):
        hg.Plan(torch.zeros((48, 4, 256), dtype=torch.uint8), torch.zeros((48, 4)))


def test_no_cpu_fallback_in_package():
    """The package's Python code never imports the oracle or the workloads generator."""
    pkg = os.path.join(ROOT, "hashed_gram_memory_amd")
    for f in glob.glob(os.path.join(pkg, "*.py")):
        text = open(f).read()
        assert "oracle" not in text.replace("oracle.", "") or "import oracle" not in text, f
        assert "import oracle" not in text and "from oracle" not in text, f
        assert "import workloads" not in text and "from workloads" not in text, f


def test_probe_validation(hg, plan):
    M = hg.measure_lib()
    L = hg.lib()
    assert M.engram_probe_read(None, 16, FAKE, None) == EINVAL
    assert M.engram_probe_read(FAKE, 17, FAKE, None) == EINVAL
    assert M.engram_probe_read(FAKE + 8, 16, FAKE, None) == EINVAL
    assert M.engram_probe_read(FAKE, 0, FAKE, None) == OK
    assert M.engram_probe_copy(FAKE, FAKE + 256, 1024, None) == EINVAL  # overlap
    assert M.engram_probe_copy(FAKE, None, 1024, None) == EINVAL
    assert M.engram_probe_copy(FAKE, FAKE + 4096, 0, None) == OK
    assert M.engram_probe_rows(None, FAKE, 1, FAKE, None) == EINVAL
    assert M.engram_probe_rows(plan, FAKE, -1, FAKE, None) == ERANGE
    assert M.engram_probe_rows(plan, FAKE, 0, FAKE, None) == OK
    assert M.engram_probe_rows(plan, FAKE, 1, FAKE + 4, None) == EINVAL


def test_lookup_validation(hg, plan):
    L = hg.lib()
    assert L.engram_lookup(None, FAKE, None, 1, 1, FAKE, None) == EINVAL
    assert L.engram_lookup(plan, FAKE, None, 0, 5, FAKE, None) == OK
    assert L.engram_lookup(plan, FAKE, None, -1, 5, FAKE, None) == EINVAL
    assert L.engram_lookup(plan, FAKE, None, 1 << 16, 1 << 15, FAKE, None) == ERANGE
    assert L.engram_lookup(plan, None, None, 1, 1, FAKE, None) == EINVAL
    assert L.engram_lookup(plan, FAKE, None, 1, 1, FAKE + 4, None) == EINVAL
    assert L.engram_lookup(plan, FAKE, FAKE + 2, 1, 1, FAKE, None) == EINVAL


def test_lookup_dedup_validation(hg, plan):
    L = hg.lib()
    G = (FAKE + 64, FAKE + 128, FAKE + 192)  # perm, offsets, n_unique
    assert L.engram_lookup_dedup(None, FAKE, None, 1, 1, *G, FAKE, None) == EINVAL
    assert L.engram_lookup_dedup(plan, FAKE, None, 0, 5, *G, FAKE, None) == OK
    assert L.engram_lookup_dedup(plan, FAKE, None, 0, 5, None, None, None, FAKE, None) == OK
    assert L.engram_lookup_dedup(plan, FAKE, None, -1, 5, *G, FAKE, None) == EINVAL
    assert L.engram_lookup_dedup(plan, FAKE, None, 1 << 16, 1 << 15, *G, FAKE, None) == ERANGE
    assert L.engram_lookup_dedup(plan, None, None, 1, 1, *G, FAKE, None) == EINVAL
    assert L.engram_lookup_dedup(plan, FAKE, None, 1, 1, *G, FAKE + 4, None) == EINVAL
    assert L.engram_lookup_dedup(plan, FAKE, FAKE + 2, 1, 1, *G, FAKE, None) == EINVAL
    for k in range(3):  # every group pointer is required and 4-byte aligned
        missing, skewed = list(G), list(G)
        missing[k] = None
        skewed[k] = G[k] + 2
        assert L.engram_lookup_dedup(plan, FAKE, None, 1, 1, *missing, FAKE, None) == EINVAL
        assert L.engram_lookup_dedup(plan, FAKE, None, 1, 1, *skewed, FAKE, None) == EINVAL


def test_plan_scale_formats(hg):
    M = hg.measure_lib()
    L = hg.lib()
    d, keep = _desc(hg, scs=[FAKE + 8 * s for s in range(48)])
    d.scale_format = 1
    st, h = _plan(hg, d)
    assert st == OK
    L.engram_plan_destroy(h)
    d, keep = _desc(hg, scs=[FAKE + 4 + 8 * s for s in range(48)])
    d.scale_format = 1
    assert _plan(hg, d)[0] == EINVAL  # block scales must be 8-byte aligned
    d, keep = _desc(hg)
    d.scale_format = 2
    assert _plan(hg, d)[0] == EUNSUPPORTED
    d, keep = _desc(hg)
    d.reserved1 = 1
    assert _plan(hg, d)[0] == EINVAL
    assert M.engram_synth_fill_e8m0(FAKE, 0, 0, 1, None) == ERANGE
    assert M.engram_synth_fill_e8m0(FAKE + 4, 16, 0, 1, None) == EINVAL
    assert M.engram_synth_fill_e8m0(FAKE, 16, 48, 1, None) == EINVAL
    assert M.engram_synth_fill_e8m0(None, 16, 0, 1, None) == EINVAL


def test_gate_io_validation(hg, plan):
    L = hg.lib()
    assert L.engram_gather_weighted(None, FAKE, 1, FAKE, FAKE, None) == EINVAL
    assert L.engram_gather_weighted(plan, FAKE, 0, FAKE, FAKE, None) == OK
    assert L.engram_gather_weighted(plan, FAKE, -1, FAKE, FAKE, None) == ERANGE
    assert L.engram_gather_weighted(plan, FAKE, 1, None, FAKE, None) == EINVAL
    assert L.engram_gather_weighted(plan, FAKE, 1, FAKE + 4, FAKE, None) == EINVAL
    assert L.engram_gather_rows(None, FAKE, 1, FAKE, None) == EINVAL
    assert L.engram_gather_rows(plan, FAKE, 0, FAKE, None) == OK
    assert L.engram_gather_rows(plan, FAKE, 1, FAKE + 8, None) == EINVAL
    assert L.engram_gather_rows(plan, FAKE, 1 << 31, FAKE, None) == ERANGE


def test_plan_vocab_map(hg):
    d, keep = _desc(hg)
    d.vocab_map = FAKE
    assert _plan(hg, d)[0] == EINVAL  # a map needs its length in vocab_size
    d.vocab_size = 1000
    st, h = _plan(hg, d)
    assert st == OK
    hg.lib().engram_plan_destroy(h)
    d.vocab_map = FAKE + 2
    assert _plan(hg, d)[0] == EINVAL


def test_probe_random_validation(hg):
    M = hg.measure_lib()
    L = hg.lib()
    assert M.engram_probe_random(None, 1 << 20, 256, 1 << 20, 1, FAKE, None) == EINVAL
    assert M.engram_probe_random(FAKE + 16, 1 << 20, 256, 1 << 20, 1, FAKE, None) == EINVAL
    assert M.engram_probe_random(FAKE, 1 << 20, 300, 1 << 20, 1, FAKE, None) == EUNSUPPORTED
    assert M.engram_probe_random(FAKE, 100, 256, 1 << 20, 1, FAKE, None) == EINVAL
    assert M.engram_probe_random(FAKE, 1 << 20, 256, 100, 1, FAKE, None) == OK  # less than one wave: nothing to do


def test_probe_records_validation(hg):
    M = hg.measure_lib()
    L = hg.lib()
    assert M.engram_probe_records(None, 1 << 20, 0, 4, 1, FAKE, None) == EINVAL
    assert M.engram_probe_records(FAKE + 16, 1 << 20, 0, 4, 1, FAKE, None) == EINVAL
    assert M.engram_probe_records(FAKE, 1 << 20, 0, 4, 1, FAKE + 4, None) == EINVAL
    assert M.engram_probe_records(FAKE, 1 << 20, 0, -1, 1, FAKE, None) == EINVAL
    assert M.engram_probe_records(FAKE, 1 << 20, 4, 4, 1, FAKE, None) == EUNSUPPORTED
    assert M.engram_probe_records(FAKE, 200, 0, 4, 1, FAKE, None) == EINVAL
    assert M.engram_probe_records(FAKE, 1 << 20, 3, 0, 1, FAKE, None) == OK


def test_gather_reduce_batched_validation(hg, plan):
    L = hg.lib()
    assert L.engram_gather_reduce_batched(None, FAKE, 1, 1, FAKE, None) == EINVAL
    assert L.engram_gather_reduce_batched(plan, FAKE, 0, 5, FAKE, None) == OK
    assert L.engram_gather_reduce_batched(plan, FAKE, 5, 0, FAKE, None) == OK
    assert L.engram_gather_reduce_batched(plan, FAKE, -1, 5, FAKE, None) == EINVAL
    assert L.engram_gather_reduce_batched(plan, FAKE, 2, -5, FAKE, None) == EINVAL
    assert L.engram_gather_reduce_batched(plan, FAKE, 1 << 16, 1 << 16, FAKE, None) == ERANGE
    assert L.engram_gather_reduce_batched(plan, None, 2, 3, FAKE, None) == EINVAL
    assert L.engram_gather_reduce_batched(plan, FAKE + 4, 2, 3, FAKE, None) == EINVAL
    assert L.engram_gather_reduce_batched(plan, FAKE, 2, 3, FAKE + 8, None) == EINVAL


def test_binding_rejects_groups_of_another_size(hg):
    """dedup(), gather_reduce() and lookup() refuse a Groups sized for another token count before any call is
    made."""
    import torch
    ids = torch.zeros((2, 50), dtype=torch.int32)
    addr = torch.zeros((100, 48), dtype=torch.int32).view(torch.uint32)
    good = hg.Groups(torch.zeros(100, dtype=torch.int32), torch.zeros(101, dtype=torch.int32),
                     torch.zeros(1, dtype=torch.int32))
    bad = [
        hg.Groups(torch.zeros(99, dtype=torch.int32), good.offsets, good.n_unique),
        hg.Groups(good.perm, torch.zeros(100, dtype=torch.int32), good.n_unique),
        hg.Groups(good.perm, good.offsets, torch.zeros(0, dtype=torch.int32)),
        hg.Groups(torch.zeros((100, 1), dtype=torch.int32), good.offsets, good.n_unique),
    ]
    for g in bad:
        with pytest.raises(ValueError, match="groups"):
            hg.dedup(None, ids, groups=g)
        with pytest.raises(ValueError, match="groups"):
            hg.gather_reduce(None, addr, groups=g)
        with pytest.raises(ValueError, match="groups"):
            hg.lookup(None, ids, groups=g)


def test_dedup_noalloc_validation(hg, plan):
    """engram_dedup_noalloc validates on the host like engram_dedup and refuses, before any launch, a batch whose
    workspace exceeds its fixed device array."""
    L = hg.lib()
    assert L.engram_dedup_noalloc(None, FAKE, None, 1, 10, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.engram_dedup_noalloc(plan, FAKE, None, -1, 10, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.engram_dedup_noalloc(plan, FAKE, None, 1, 10, None, FAKE, FAKE, None) == EINVAL
    assert L.engram_dedup_noalloc(plan, FAKE, None, 1, 10, FAKE, FAKE + 2, FAKE, None) == EINVAL
    assert L.engram_dedup_noalloc(plan, FAKE, None, 1 << 11, (1 << 11) + 1, FAKE, FAKE, FAKE, None) == ERANGE
    # a batch whose workspace is above the fixed size: the plan fixture has vocab_size 0 (31-bit ids, the widest keys)
    b = ctypes.c_size_t()
    n = 1 << 22
    assert L.engram_dedup_workspace(plan, n, ctypes.byref(b)) == OK and b.value > hg.DEDUP_SCRATCH_BYTES
    assert L.engram_dedup_noalloc(plan, FAKE, None, 1, n, FAKE, FAKE, FAKE, None) == EWORKSPACE
    # the size the fixed array is stated to hold under any plan
    assert L.engram_dedup_workspace(plan, 524288, ctypes.byref(b)) == OK and b.value <= hg.DEDUP_SCRATCH_BYTES


def test_check_inputs_validation(hg, plan):
    L = hg.lib()
    assert L.engram_check_inputs(None, FAKE, None, 1, 1, FAKE, 1, FAKE, None) == EINVAL
    assert L.engram_check_inputs(plan, FAKE, None, 1, 1, FAKE, 1, None, None) == EINVAL
    assert L.engram_check_inputs(plan, FAKE, None, 1, 1, FAKE, 1, FAKE + 2, None) == EINVAL
    assert L.engram_check_inputs(plan, FAKE + 2, None, 1, 1, None, 0, FAKE, None) == EINVAL
    assert L.engram_check_inputs(plan, None, FAKE, 1, 1, None, 0, FAKE, None) == EINVAL  # history needs ids
    assert L.engram_check_inputs(plan, None, None, 0, 0, FAKE + 4, 1, FAKE, None) == EINVAL  # addr 16-byte aligned
    assert L.engram_check_inputs(plan, FAKE, None, -1, 1, None, 0, FAKE, None) == EINVAL
    assert L.engram_check_inputs(plan, FAKE, None, 1 << 16, 1 << 15, None, 0, FAKE, None) == ERANGE
    assert L.engram_check_inputs(plan, None, None, 0, 0, FAKE, -1, FAKE, None) == ERANGE
