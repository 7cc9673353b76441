"""The allocation-free embedding-gradient scatter against the workspace one.

mlb_prim_embed_scatter_noalloc keeps its sort keys in the library's static
device array instead of a caller workspace. Called through the C ABI twice in
a row (the second call smaller, so the array still holds the first call's
keys), it must give the workspace entry point's bits, which are the oracle's
(each row a left fold over its positions in increasing order).
"""
import ctypes as C

import numpy as np
import pytest

import oracle
from bitwise_reproducible_fp32_amd import inputs as I
from gpu_util import assert_bits, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mlb():
    import bitwise_reproducible_fp32_amd as m
    return m


def run_both(mlb, ids, dh, d, V, dE0):
    import torch
    L = mlb.lib()
    s = torch.cuda.current_stream().cuda_stream
    N = ids.size
    i_d, h_d = dev(ids), dev(dh)
    ws = torch.empty(2 * 8192 * 8, dtype=torch.uint8, device="cuda")
    a, b = dev(dE0), dev(dE0)
    assert L.mlb_prim_embed_scatter(i_d.data_ptr(), h_d.data_ptr(), N, d, V, a.data_ptr(), ws.data_ptr(),
                                    ws.numel(), s) == 0
    rc = L.mlb_prim_embed_scatter_noalloc(i_d.data_ptr(), h_d.data_ptr(), N, d, V, b.data_ptr(), s)
    assert rc == 0, L.mlb_last_error_message().decode()
    return host(a), host(b)


def test_noalloc_scatter_matches_workspace_entry_point(mlb):
    V, d = 50257, 768
    rng = np.random.default_rng(5)
    for N in (8192, 1000):            # a full-size call, then a smaller one over the same array
        ids = I.zipf_ids(N, V, [5, N])
        ids[::97] = V + 3             # out-of-range ids are skipped by both
        dh = rng.uniform(-1, 1, (N, d)).astype(np.float32)
        dE0 = np.zeros((V, d), np.float32)
        dE0[ids[ids < V][:50]] = rng.uniform(-1, 1, (50, d)).astype(np.float32)
        want_ws, got = run_both(mlb, ids, dh, d, V, dE0)
        assert_bits(f"N={N} noalloc vs workspace", got, want_ws)
        keep = ids < V
        want = oracle.embed_scatter(ids[keep], dh[keep], dE0)
        assert_bits(f"N={N} noalloc vs oracle", got, want)


def test_noalloc_scatter_refuses_beyond_its_array(mlb):
    import torch
    L = mlb.lib()
    s = torch.cuda.current_stream().cuda_stream
    ids = torch.zeros(8193, dtype=torch.int32, device="cuda")
    dh = torch.zeros(8193 * 4, dtype=torch.float32, device="cuda")
    dE = torch.zeros(16 * 4, dtype=torch.float32, device="cuda")
    rc = L.mlb_prim_embed_scatter_noalloc(ids.data_ptr(), dh.data_ptr(), 8193, 4, 16, dE.data_ptr(), s)
    assert mlb.STATUS[rc] == "MLB_E_UNSUPPORTED"
    assert "8192" in L.mlb_last_error_message().decode()
    rc = L.mlb_prim_embed_scatter_noalloc(ids.data_ptr(), dh.data_ptr(), 0, 4, 16, dE.data_ptr(), s)
    assert rc == 0
    assert np.all(host(dE) == 0)
