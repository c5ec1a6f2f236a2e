"""The CPU oracle against facts that do not come from the oracle itself."""
import os

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_byte_model.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = v
    return vals


def test_windows_worked_examples():
    pins.check_windows(oracle.windows)


def test_windows_reject_negative_ids():
    with pytest.raises(ValueError):
        oracle.windows(np.array([[1, -2]], np.int32))


def test_splitmix64_known_answers():
    pins.check_splitmix(oracle.splitmix64)


def test_multipliers():
    pins.check_multipliers(oracle.multipliers)


def test_hash_properties():
    pins.check_hash(oracle.hash_addresses, oracle.multipliers)


def test_hash_rejects_bad_rows():
    w = np.zeros((1, 4), np.int64)
    m = oracle.multipliers()
    for rows in ([0] * 48, [(1 << 32) + 1] * 48, [4] * 47):
        with pytest.raises(ValueError):
            oracle.hash_addresses(w, m, rows)


def test_e4m3_decode_against_torch_and_textbook():
    pins.check_decode(oracle.E4M3_TABLE)


def test_gather_reduce_closed_forms():
    pins.check_gather_reduce(oracle.gather_reduce)


def test_dedup_properties_and_python_sort():
    pins.check_dedup(oracle.dedup)


def test_geometry_matches_pages_byte_model():
    g = _golden()
    orders = tuple(int(x) for x in g["ngram_orders"].split(","))
    assert orders == oracle.ORDERS
    assert int(g["modules"]) == oracle.N_MODULES
    assert int(g["heads_per_module_and_order"]) == oracle.N_HEADS
    assert int(g["rows_per_layer"]) == oracle.ROWS_PER_MODULE
    assert int(g["rows_per_token"]) == oracle.N_SUB
    assert int(g["row_fp8_bytes"]) == oracle.ROW_BYTES
    # the oracle emits exactly one address per (module, order, head), 48 per token
    win = oracle.windows(np.arange(10, dtype=np.int32).reshape(1, 10))
    addr = oracle.hash_addresses(win, oracle.multipliers(), [1 << 20] * 48)
    assert addr.shape == (10, int(g["rows_per_token"]))
    # per-token bytes: 48 x (256 + 8) = 12,672, ~12 KB
    per_tok = oracle.N_SUB * (oracle.ROW_BYTES + int(g["row_scale_bytes"]))
    assert per_tok == int(g["bytes_per_token"])
    # "about 12 KB" is the FP8 rows alone: 48 x 256 B = 12 KiB
    rows_bytes = oracle.N_SUB * oracle.ROW_BYTES
    assert rows_bytes / 1024 == int(g["approx_kb_per_token"])
    # 10 tok/s x 12 KiB = 120 KiB/s; 2,000 tok/s x 12,672 B = ~25 MB/s; 128K tokens = ~1.7 GB
    assert int(g["decode_tokens_per_s"]) * rows_bytes / 1024 == int(g["decode_read_kb_per_s"])
    assert round(int(g["aggregate_tokens_per_s"]) * per_tok / 1e6) == int(g["aggregate_mb_per_s"])
    assert round(int(g["prompt_tokens"]) * per_tok / 1e9, 1) == float(g["prompt_gb"])
    # 2 tables x ~384M rows x 256 = 196.6B parameters; 24 sub-tables of 2^24 rows is within 5% of ~384M rows
    params = int(g["tables"]) * int(g["approx_rows_per_table_millions"]) * 1e6 * oracle.ROW_BYTES
    assert round(params / 1e9, 1) == float(g["table_params_billions"])
    rows_full = oracle.ROWS_PER_MODULE * (1 << 24)
    assert abs(rows_full / (int(g["approx_rows_per_table_millions"]) * 1e6) - 1) < 0.05


def test_oracle_is_exact_in_float64():
    """For the synthetic scale grid the float64 sums carry no rounding: sum order is irrelevant."""
    import workloads
    rng = np.random.default_rng(5)
    tabs, scs = workloads.dense_tables(77, 64)
    addr = rng.integers(0, 64, size=(50, 48)).astype(np.uint32)
    out, _ = oracle.gather_reduce(tabs, scs, addr)
    # reverse the sub-table order inside each module: same bits
    rev_t = [tabs[24 * (s // 24) + 23 - s % 24] for s in range(48)]
    rev_s = [scs[24 * (s // 24) + 23 - s % 24] for s in range(48)]
    rev_a = np.stack([addr[:, 24 * (s // 24) + 23 - s % 24] for s in range(48)], axis=1)
    out2, _ = oracle.gather_reduce(rev_t, rev_s, rev_a)
    assert np.array_equal(out, out2)


def test_e8m0_decode_against_torch():
    pins.check_e8m0(oracle.E8M0_TABLE)


def test_gather_reduce_e8m0_closed_forms():
    pins.check_gather_reduce_e8m0(lambda t, s, a: oracle.gather_reduce(t, s, a, "e8m0_block32"))


def test_scale_format_rejected():
    with pytest.raises(ValueError):
        oracle.gather_reduce([np.zeros((1, 256), np.uint8)] * 48, [np.ones(1, np.float32)] * 48,
                             np.zeros((1, 48), np.uint32), "bf16")


def test_gate_inputs():
    pins.check_gate_inputs(oracle.gather_rows, oracle.gather_weighted, oracle.gather_reduce)


def test_windows_vocab_map():
    pins.check_windows_map(oracle.windows)


def test_vocab_map_merges_rows():
    """Ids the map folds together hash to the same rows; the others do not."""
    import workloads
    vmap = workloads.vocab_map(3, vocab=1000, compressed=600)
    assert vmap.max() < 600 and len(np.unique(vmap)) == 600
    a, b = [int(x) for x in np.flatnonzero(vmap == vmap[900])[:2]]
    ids = np.array([[a, 1, 2], [b, 1, 2]], np.int32)
    addr = oracle.hash_addresses(oracle.windows(ids, None, vmap), oracle.multipliers(), [1 << 20] * 48)
    assert np.array_equal(addr[0], addr[3]) and np.array_equal(addr[1], addr[4])
    raw = oracle.hash_addresses(oracle.windows(ids, None), oracle.multipliers(), [1 << 20] * 48)
    assert not np.array_equal(raw[0], raw[3])


def test_prime_rows():
    import workloads
    p = workloads.prime_rows(5, below=100)
    assert p == [97, 89, 83, 79, 73]
