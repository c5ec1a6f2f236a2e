"""engram_dedup_noalloc (the dedup entry point that allocates nothing) against engram_dedup and the oracle: two
calls in a row through the C ABI, the second with a smaller batch, each bit-exact."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import dummy_plan, lib, to_dev_ids

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _groups(n_tok):
    return lib().Groups(torch.full((n_tok,), -7, dtype=torch.int32, device="cuda"),
                        torch.full((n_tok + 1,), -7, dtype=torch.int32, device="cuda"),
                        torch.full((1,), -7, dtype=torch.int32, device="cuda"))


def _noalloc(plan, d_ids, d_hist, g):
    n_seq, seq_len = d_ids.shape
    st = lib().lib().engram_dedup_noalloc(plan.handle, d_ids.data_ptr(), None if d_hist is None else d_hist.data_ptr(),
                                          n_seq, seq_len, g.perm.data_ptr(), g.offsets.data_ptr(),
                                          g.n_unique.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib().lib().engram_status_string(st)


def _host(g, nu=None):
    nu = int(g.n_unique.item()) if nu is None else nu
    return nu, g.perm.cpu().numpy(), g.offsets[:nu + 1].cpu().numpy()


def test_noalloc_equals_dedup_two_calls():
    plan = dummy_plan(4096, workloads.VOCAB)
    rng = np.random.default_rng(707)
    cases = [  # the second batch is smaller and has a history
        (workloads.zipf_ids(rng, 16 * 6000).reshape(16, 6000), None),
        (workloads.zipf_ids(rng, 3 * 777).reshape(3, 777), workloads.zipf_ids(rng, 9).reshape(3, 3)),
    ]
    for call, (ids, hist) in enumerate(cases):
        _say(f"call {call}: dedup_noalloc {ids.shape[0]} x {ids.shape[1]}, history={hist is not None}")
        d_ids, d_hist = to_dev_ids(ids, hist)
        n_tok = ids.size
        g_fixed, g_ws = _groups(n_tok), _groups(n_tok)
        _noalloc(plan, d_ids, d_hist, g_fixed)
        ws = torch.empty(lib().dedup_workspace_bytes(plan, n_tok), dtype=torch.uint8, device="cuda")
        lib().dedup(plan, d_ids, d_hist, workspace=ws, groups=g_ws)
        torch.cuda.synchronize()
        nu, perm, off = _host(g_fixed)
        nu_ws, perm_ws, off_ws = _host(g_ws)
        assert nu == nu_ws
        assert np.array_equal(perm, perm_ws)
        assert np.array_equal(off, off_ws)
        want_perm, want_off, want_nu = oracle.dedup(oracle.windows(ids, hist))
        assert nu == want_nu
        assert np.array_equal(perm, want_perm)
        assert np.array_equal(off, want_off)


def test_noalloc_refuses_a_batch_beyond_its_array():
    """A batch whose workspace exceeds the fixed array is refused on the host, with the outputs untouched."""
    plan = dummy_plan(4096, 0)
    n = 1 << 22
    need = lib().dedup_workspace_bytes(plan, n)
    assert need > lib().DEDUP_SCRATCH_BYTES
    d_ids = torch.zeros((1, n), dtype=torch.int32, device="cuda")
    g = _groups(n)
    st = lib().lib().engram_dedup_noalloc(plan.handle, d_ids.data_ptr(), None, 1, n, g.perm.data_ptr(),
                                          g.offsets.data_ptr(), g.n_unique.data_ptr(), None)
    assert st == -3  # ENGRAM_EWORKSPACE
    torch.cuda.synchronize()
    assert int(g.n_unique.item()) == -7
