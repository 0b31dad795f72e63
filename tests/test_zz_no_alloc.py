"""dsa_topk_static (the top-k entry point that allocates nothing: split rows keep
their survivors in the library's static device array) against dsa_topk with a
caller workspace, both through the C ABI: bit-exact indices on consecutive
calls, each later one smaller than the one before (the array keeps the
previous call's contents), on split and unsplit shapes."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, say
import long_context_sparse_fp8_amd as dsa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return dsa.lib()


def _inputs(n_q, ld, k, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((n_q, ld)).astype(np.float32)
    s[::3] = np.round(s[::3] * 2) / 2                            # ties in every third row
    pos = rng.integers(0, ld, n_q).astype(np.int32)
    pos[:3] = [ld - 1, min(ld - 1, 2 * k), min(ld - 1, k - 1)]
    return s, pos


def _run(L, s, pos, k, static):
    n_q, ld = s.shape
    sd, pd = torch.from_numpy(s).to(DEV), torch.from_numpy(pos).to(DEV)
    idx = torch.full((n_q, k), -7, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if static:
        rc = L.dsa_topk_static(sd.data_ptr(), ld, pd.data_ptr(), n_q, k, idx.data_ptr(), stream)
    else:
        need = L.dsa_topk_workspace_size(n_q, ld, k)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        rc = L.dsa_topk(sd.data_ptr(), ld, pd.data_ptr(), n_q, k, idx.data_ptr(), ws.data_ptr() if need else None,
                        need, stream)
    assert rc == 0, L.dsa_last_error().decode()
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def test_static_workspace_topk_matches_workspace_topk(L):
    # decreasing sizes: 64 long rows in 4 parts (4 MiB of survivors), 16 rows in
    # 8 parts, k = 1 on short split rows, then rows that are not split at all
    cases = [(64, 131072, 2048), (16, 40000, 333), (40, 100, 1), (300, 5000, 2048)]
    for i, (n_q, ld, k) in enumerate(cases):
        s, pos = _inputs(n_q, ld, k, 900 + i)
        split = L.dsa_topk_workspace_size(n_q, ld, k)
        say(f"[topk static] call {i}: {n_q} rows x {ld}, k={k}, split workspace {split} bytes")
        got = _run(L, s, pos, k, static=True)
        want = _run(L, s, pos, k, static=False)
        np.testing.assert_array_equal(got, want)
        if n_q * ld <= 2_000_000:
            np.testing.assert_array_equal(got, oracle.topk(s, pos, k))


def test_static_workspace_topk_repeated_calls_keep_no_state(L):
    """The same small call before and after a large one gives the same indices."""
    s, pos = _inputs(16, 40000, 333, 950)
    first = _run(L, s, pos, 333, static=True)
    big_s, big_pos = _inputs(128, 70000, 2048, 951)
    np.testing.assert_array_equal(_run(L, big_s, big_pos, 2048, static=True),
                                  _run(L, big_s, big_pos, 2048, static=False))
    np.testing.assert_array_equal(_run(L, s, pos, 333, static=True), first)


def test_static_workspace_topk_rejects_bad_arguments_on_the_host(L):
    A = ctypes.c_void_p(0x1000)
    assert L.dsa_topk_static(A, 100, A, 4, 0, A, None) == 3
    assert L.dsa_topk_static(None, 100, A, 4, 16, A, None) == 1
    assert L.dsa_topk_static(A, 100, A, 4, 16, ctypes.c_void_p(0x1004), None) == 4
    assert L.dsa_topk_static(None, 100, None, 0, 16, None, None) == 0
