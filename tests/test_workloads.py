"""The seeded synthetic inputs: shapes, ranges and distributions."""
import numpy as np

import workloads


def test_workload_shapes():
    exp = {1: (1, 512, 4096), 2: (64, 1, 1 << 20), 3: (1, 32768, 1 << 22),
           4: (1, 131072, 1 << 24), 5: (64, 8192, 1 << 24)}
    for k, (s, t, r) in exp.items():
        w = workloads.WORKLOADS[k]
        assert (w.n_seq, w.seq_len, w.rows) == (s, t, r)
        assert w.table_seed == 1000 + k and w.token_seed == 2000 + k


def test_ids_ranges_and_structure():
    ids, hist = workloads.make_ids(workloads.WORKLOADS[1])
    assert ids.dtype == np.int32 and hist is None and ids.min() >= 0 and ids.max() < 1024
    ids, hist = workloads.make_ids(workloads.WORKLOADS[2])
    assert ids.shape == (64, 1) and hist.shape == (64, 3)
    ids, hist = workloads.make_ids(workloads.WORKLOADS[5])
    assert ids.shape == (64, 8192) and hist is None
    assert (ids[:, :4096] == ids[0, :4096]).all()  # shared prefix
    assert not (ids[:, 4096:] == ids[0, 4096:]).all(axis=1)[1:].any()  # independent suffixes
    # deterministic
    again, _ = workloads.make_ids(workloads.WORKLOADS[5])
    assert np.array_equal(ids, again)


def test_zipf_frequencies():
    rng = np.random.Generator(np.random.PCG64(1))
    ids = workloads.zipf_ids(rng, 400_000)
    assert ids.min() >= 0 and ids.max() < workloads.VOCAB
    ranks = np.arange(1, workloads.VOCAB + 1, dtype=np.float64)
    p = ranks ** -1.1
    p /= p.sum()
    cnt = np.bincount(ids, minlength=workloads.VOCAB)
    for r in range(10):  # the head of the distribution within 4 sigma
        exp = p[r] * ids.size
        assert abs(cnt[r] - exp) < 4 * np.sqrt(exp) + 1, r


def test_table_generator_codes_and_scales():
    codes, scales = workloads.table_range(1234, 7, 1000, 2000)
    assert codes.shape == (2000, 256) and scales.shape == (2000,)
    assert not np.isin(codes, [0x7F, 0xFF]).any()  # no NaN codes
    cnt = np.bincount(codes.ravel(), minlength=256)
    valid = np.setdiff1d(np.arange(256), [0x7F, 0xFF])
    exp = codes.size / 254
    chi2 = (((cnt[valid] - exp) ** 2) / exp).sum()
    assert chi2 < 400  # 253 dof
    assert scales.min() >= 0.5 and scales.max() < 2.0
    k = scales.astype(np.float64) * 2 ** 23
    assert np.array_equal(k, np.round(k))  # exact k * 2^-23
    # row-wise and range-wise generation agree; other sub-tables and seeds differ
    c2, s2 = workloads.table_rows(1234, 7, np.arange(1000, 3000))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    c3, _ = workloads.table_range(1234, 8, 1000, 2000)
    c4, _ = workloads.table_range(1235, 7, 1000, 2000)
    assert (c3 != codes).mean() > 0.9 and (c4 != codes).mean() > 0.9


def test_sparse_host_tables_hold_requested_rows():
    t = workloads.SparseHostTables(99, 1 << 24)  # 192 GiB of address space, a few pages resident
    addr = np.random.default_rng(0).integers(0, 1 << 24, size=(5, 48)).astype(np.uint32)
    t.materialise(addr)
    for s in (0, 17, 47):
        c, sc = workloads.table_rows(99, s, addr[:, s])
        assert np.array_equal(t.tables[s][addr[:, s].astype(np.int64)], c)
        assert np.array_equal(t.scales[s][addr[:, s].astype(np.int64)], sc)
    t.close()


def test_e8m0_generator():
    e = workloads.e8m0_range(42, 5, 100, 3000)
    assert e.shape == (3000, 8) and e.min() >= 120 and e.max() <= 134
    assert len(np.unique(e)) == 15
    assert np.array_equal(workloads.e8m0_rows(42, 5, np.arange(100, 3100)), e)
    t = workloads.SparseHostTables(42, 1 << 20, "e8m0_block32")
    addr = np.random.default_rng(1).integers(0, 1 << 20, size=(4, 48)).astype(np.uint32)
    t.materialise(addr)
    assert np.array_equal(t.scales[5][addr[:, 5].astype(np.int64)], workloads.e8m0_rows(42, 5, addr[:, 5]))
    t.close()
