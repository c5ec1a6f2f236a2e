"""engram_gather_reduce_batched: the direct-mode gather visiting a batch in tiles of positions gives the flat
gather's result bitwise, for every shape (ragged last tiles, sequences shorter than a tile, one sequence, the
2^24-item launch boundary) and both scale formats."""
import numpy as np
import pytest
import torch

import workloads
from gpu_support import lib, small_device_tables, to_dev_ids

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("fmt", ["f32_row", "e8m0_block32"])
@pytest.mark.parametrize("n_seq,seq_len,shared", [
    (1, 1000, 0), (3, 5, 0), (5, 77, 30), (64, 300, 128), (2, 64, 64), (7, 129, 0), (64, 1, 0),
])
def test_batched_equals_flat(fmt, n_seq, seq_len, shared):
    _say(f"batched gather {n_seq}x{seq_len} shared={shared} {fmt}")
    R = 4096
    host_t, host_c = workloads.dense_tables(31, R, fmt)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c, scale_format=fmt)
    rng = np.random.default_rng(n_seq * 1000 + seq_len)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len)).astype(np.int32)
    if shared:
        ids[:, :shared] = ids[0, :shared]
    d_ids, _ = to_dev_ids(ids, None)
    addr = lib().hash(plan, d_ids)
    flat = lib().gather_reduce(plan, addr)
    batched = torch.full_like(flat, float("nan"))
    lib().gather_reduce_batched(plan, addr, n_seq, out=batched)
    fused = lib().lookup(plan, d_ids)
    torch.cuda.synchronize()
    assert torch.equal(batched, flat)
    assert torch.equal(fused, flat)


def _token_checksums(out):
    step = 1 << 20
    return torch.cat([out[i:i + step].reshape(-1, 512).double().sum(dim=1) for i in range(0, out.shape[0], step)])


def test_batched_across_the_chunk_boundary():
    """Two sequences of 2^23 + 40 tokens: the batched gather splits its grid at 2^24 items, where the last,
    40-position tile begins; per-token checksums and a sample of tokens equal the flat gather's."""
    n_seq, seq_len = 2, (1 << 23) + 40
    _say(f"batched gather, {n_seq} x {seq_len} tokens")
    R = 512
    host_t, host_c = workloads.dense_tables(810, R)
    t, c = small_device_tables(host_t, host_c)
    plan = lib().Plan(t, c)
    rng = np.random.default_rng(26)
    ids = rng.integers(0, 129280, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    d_ids, _ = to_dev_ids(ids, None)
    n_tok = n_seq * seq_len
    sample = torch.from_numpy(np.unique(np.concatenate([
        np.arange(0, 130), np.arange(seq_len - 100, seq_len + 100), np.arange(n_tok - 100, n_tok),
        rng.integers(0, n_tok, 4000)]))).cuda()
    addr = lib().hash(plan, d_ids)
    out = lib().gather_reduce_batched(plan, addr, n_seq)
    batched_sum = _token_checksums(out)
    batched_sample = out[sample].clone()
    lib().gather_reduce(plan, addr, out=out)
    torch.cuda.synchronize()
    flat_sum = _token_checksums(out)
    flat_sample = out[sample].clone()
    del addr, out
    torch.cuda.empty_cache()
    assert torch.equal(batched_sample, flat_sample)
    assert torch.equal(batched_sum, flat_sum)
