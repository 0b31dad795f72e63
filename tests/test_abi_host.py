"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/dsa.h declares, and rejects bad arguments on the
host before anything is enqueued (each error path is forced from the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    import long_context_sparse_fp8_amd as dsa
    return dsa.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["dsa_indexer_cache_store", "dsa_kv_cache_store", "dsa_indexer_scores", "dsa_topk",
              "dsa_sparse_mla_prefill", "dsa_sparse_mla_decode", "dsa_topk_workspace_size",
              "dsa_sparse_mla_decode_workspace_size", "dsa_abi_version", "dsa_status_string", "dsa_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n
    assert L.dsa_abi_version() == 1


def test_status_strings(L):
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(3) == b"DSA_ERR_UNSUPPORTED"
    assert L.dsa_status_string(99) == b"DSA_ERR_UNKNOWN"


P = ctypes.c_void_p
A = P(0x1000)          # aligned non-null dummy pointer (never dereferenced: validation fails first)
MIS = P(0x1004)        # misaligned


def _err(L):
    return L.dsa_last_error().decode()


def test_indexer_scores_validation(L):
    # unsupported (h_i, d_i)
    rc = L.dsa_indexer_scores(A, A, A, 32, A, A, 10, A, 4, A, A, 5, 32, 128, A, 100, None)
    assert rc == 3 and "h_i" in _err(L)
    # null pointer
    rc = L.dsa_indexer_scores(None, A, A, 64, A, A, 10, A, 4, A, A, 5, 64, 128, A, 100, None)
    assert rc == 1 and "q_fp8" in _err(L)
    # misaligned
    rc = L.dsa_indexer_scores(A, A, A, 64, A, A, 10, A, 4, A, A, 5, 64, 128, MIS, 100, None)
    assert rc == 4 and "scores" in _err(L)
    # bad leading dimensions / counts
    assert L.dsa_indexer_scores(A, A, A, 7, A, A, 10, A, 4, A, A, 5, 64, 128, A, 100, None) == 2
    assert L.dsa_indexer_scores(A, A, A, 64, A, A, 10, A, 0, A, A, 5, 64, 128, A, 100, None) == 2
    assert L.dsa_indexer_scores(A, A, A, 64, A, A, 10, A, 4, A, A, -1, 64, 128, A, 100, None) == 2
    # n_q == 0 is a no-op, even with NULL pointers
    assert L.dsa_indexer_scores(None, None, None, 64, None, None, 10, None, 4, None, None, 0, 64, 128,
                                None, 100, None) == 0


def test_topk_validation(L):
    assert L.dsa_topk(A, 100, A, 4, 0, A, None, 0, None) == 3
    assert L.dsa_topk(A, 100, A, 4, 2049, A, None, 0, None) == 3
    assert L.dsa_topk(A, 0, A, 4, 16, A, None, 0, None) == 2
    assert L.dsa_topk(A, 262144, A, 4, 16, MIS, None, 0, None) == 4   # longest row accepted; MIS trips next
    assert L.dsa_topk(A, 262145, A, 4, 16, A, None, 0, None) == 3    # beyond DSA_MAX_TOPK_ROW
    assert L.dsa_topk(None, 100, A, 4, 16, A, None, 0, None) == 1
    assert L.dsa_topk(A, 100, A, 4, 16, MIS, None, 0, None) == 4
    assert L.dsa_topk_workspace_size(4, 100, 16) == 0
    # few long rows split over workgroups: survivors (score + index) per part
    assert L.dsa_topk_workspace_size(64, 131072, 2048) == 64 * 4 * 2048 * 8 + 256
    assert L.dsa_topk_workspace_size(16, 131072, 2048) == 16 * 8 * 2048 * 8 + 256
    assert L.dsa_topk_workspace_size(128, 131072, 2048) == 128 * 4 * 2048 * 8 + 256   # parts of <= 32K
    assert L.dsa_topk_workspace_size(128, 32768, 2048) == 128 * 2 * 2048 * 8 + 256
    assert L.dsa_topk_workspace_size(300, 131072, 2048) == 0


def test_indexer_topk_validation(L):
    """The fused indexer -> top-k call: decode form only, its workspace size,
    the two calls' shape checks."""
    per_row = (2048 + 16) * 4 + (262144 // 32 + 2 * 8192) * 4   # zero region + bitmap and candidate list
    assert per_row == 106560
    assert L.dsa_indexer_topk_workspace_size(64) == 64 * per_row
    assert L.dsa_indexer_topk_workspace_size(0) == 0
    ws = 64 * per_row
    args = lambda **kw: [kw.get("q", A), A, A, kw.get("w_ld", 64), A, A, 10, A, 4, A, A, kw.get("n_q", 64),
                         kw.get("h_i", 64), 128, kw.get("scores", A), kw.get("ld", 1000), kw.get("k", 2048),
                         A, kw.get("ws", A), kw.get("ws_bytes", ws), None]
    assert L.dsa_indexer_topk(*args(n_q=257)) == 3 and "decode form" in _err(L)
    assert L.dsa_indexer_topk(*args(h_i=32)) == 3
    assert L.dsa_indexer_topk(*args(k=0)) == 3
    assert L.dsa_indexer_topk(*args(k=2049)) == 3
    assert L.dsa_indexer_topk(*args(ld=262145)) == 3
    assert L.dsa_indexer_topk(*args(ld=0)) == 2
    assert L.dsa_indexer_topk(*args(w_ld=7)) == 2
    assert L.dsa_indexer_topk(*args(n_q=-1)) == 2
    assert L.dsa_indexer_topk(*args(q=None)) == 1
    assert L.dsa_indexer_topk(*args(scores=MIS)) == 4
    assert L.dsa_indexer_topk(*args(ws_bytes=ws - 1)) == 5
    assert L.dsa_indexer_topk(*args(ws=None)) == 1
    assert L.dsa_indexer_topk(*args(ws=MIS)) == 4
    # n_q == 0 is a no-op, even with NULL pointers
    assert L.dsa_indexer_topk(None, None, None, 64, None, None, 10, None, 4, None, None, 0, 64, 128, None, 1000,
                              2048, None, None, 0, None) == 0


def test_mla_validation(L):
    f = ctypes.c_float(1 / 24)
    args = lambda **kw: [kw.get("q", A), A, kw.get("kvs", A), kw.get("dt", 0), kw.get("n_slots", 100), A,
                         kw.get("ld", 100), A, A, kw.get("n_q", 4), kw.get("h", 128), kw.get("k", 2048),
                         kw.get("sm", f), A, kw.get("lse", None)]
    assert L.dsa_sparse_mla_prefill(*args(h=20), None) == 3   # head counts are multiples of 8
    assert L.dsa_sparse_mla_prefill(*args(h=0), None) == 3
    assert L.dsa_sparse_mla_prefill(*args(h=144), None) == 3
    assert L.dsa_sparse_mla_prefill(*args(k=0), None) == 3
    assert L.dsa_sparse_mla_prefill(*args(k=4096), None) == 3
    assert L.dsa_sparse_mla_prefill(*args(dt=5), None) == 3
    assert L.dsa_sparse_mla_prefill(*args(n_slots=0), None) == 2
    assert L.dsa_sparse_mla_prefill(*args(sm=ctypes.c_float(0.0)), None) == 2
    assert L.dsa_sparse_mla_prefill(*args(q=None), None) == 1
    assert L.dsa_sparse_mla_prefill(*args(dt=1, kvs=None), None) == 1
    assert L.dsa_sparse_mla_prefill(*args(lse=MIS), None) == 4
    # one workgroup per (query, 32 heads) needs no workspace: the automatic choice
    # when queries x head groups fill half the device
    assert L.dsa_sparse_mla_decode_workspace_size(64, 128, 2048, 0) == 0
    assert L.dsa_sparse_mla_decode_workspace_size(64, 128, 2048, 1) == 0
    assert L.dsa_sparse_mla_decode_workspace_size(8, 128, 2048, 0) > 0      # few queries: split index lists
    need = L.dsa_sparse_mla_decode_workspace_size(64, 128, 2048, 4)
    assert need == 64 * 4 * 128 * 512 * 4 + ((64 * 4 * 128 * 4 + 255) // 256) * 256 + 256
    assert L.dsa_sparse_mla_decode(*args(n_q=64), 4, A, need - 1, None) == 5
    assert L.dsa_sparse_mla_decode(*args(n_q=64), 33, A, need, None) == 3
    assert L.dsa_sparse_mla_decode(*args(n_q=64), 4, None, need, None) == 1


def test_cache_store_validation(L):
    assert L.dsa_indexer_cache_store(A, A, A, 10, 96, A, A, 4, None) == 3
    assert L.dsa_indexer_cache_store(A, A, A, -1, 128, A, A, 4, None) == 2
    assert L.dsa_indexer_cache_store(None, A, A, 10, 128, A, A, 4, None) == 1
    assert L.dsa_indexer_cache_store(None, None, None, 0, 128, None, None, 4, None) == 0
    assert L.dsa_kv_cache_store(A, A, 10, 2, A, A, 100, None) == 3
    assert L.dsa_kv_cache_store(A, A, 10, 1, A, None, 100, None) == 1
    assert L.dsa_kv_cache_store(A, MIS, 10, 0, A, None, 100, None) == 4


def test_combined_cache_store_validation(L):
    """dsa_cache_store applies the checks of both stores, before anything is
    enqueued; a zero count makes that side's pointers optional."""
    st = L.dsa_cache_store
    # (k, k_scale, key_slot, n_keys, d_i, key_cache, key_scale, n_pages,
    #  kv, kv_slot, n_kv, dt, kv_cache, kv_scale, n_slots, stream)
    assert st(None, None, None, 0, 128, None, None, 4, None, None, 0, 0, None, None, 10, None) == 0
    assert st(None, None, None, 0, 96, None, None, 4, None, None, 0, 0, None, None, 10, None) == 3     # d_i
    assert st(None, None, None, 0, 128, None, None, 4, None, None, 0, 5, None, None, 10, None) == 3    # dtype
    assert st(A, A, A, -1, 128, A, A, 4, A, A, 1, 0, A, None, 10, None) == 2
    assert st(A, A, A, 1, 128, A, A, 4, A, A, -1, 0, A, None, 10, None) == 2
    assert st(A, A, A, 1, 128, A, A, -1, None, None, 0, 0, None, None, 10, None) == 2               # n_pages
    assert st(None, A, A, 10, 128, A, A, 4, None, None, 0, 0, None, None, 10, None) == 1             # keys stored
    assert st(A, A, A, 10, 128, A, None, 4, None, None, 0, 0, None, None, 10, None) == 1
    assert st(None, None, None, 0, 128, None, None, 4, A, A, 10, 1, A, None, 10, None) == 1          # FP8: kv_scale
    assert st(None, None, None, 0, 128, None, None, 4, A, MIS, 10, 0, A, None, 10, None) == 4        # misaligned


def test_zero_counts_enqueue_nothing(L):
    """n = 0 / n_q = 0: OK with NULL data pointers (no device needed), while the
    shape and support checks still apply."""
    f = ctypes.c_float(1 / 24)
    assert L.dsa_indexer_cache_store(None, None, None, 0, 128, None, None, 4, None) == 0
    assert L.dsa_indexer_cache_store(None, None, None, 0, 96, None, None, 4, None) == 3
    assert L.dsa_kv_cache_store(None, None, 0, 0, None, None, 10, None) == 0
    assert L.dsa_kv_cache_store(None, None, 0, 1, None, None, 10, None) == 0
    assert L.dsa_kv_cache_store(None, None, 0, 7, None, None, 10, None) == 3
    assert L.dsa_indexer_scores(None, None, None, 0, None, None, 10, None, 4, None, None, 0, 64, 128,
                                None, 100, None) == 0
    assert L.dsa_topk(None, 100, None, 0, 16, None, None, 0, None) == 0
    assert L.dsa_topk(None, 100, None, 0, 0, None, None, 0, None) == 3
    for fn in (L.dsa_sparse_mla_prefill,):
        assert fn(None, None, None, 0, 100, None, 100, None, None, 0, 128, 2048, f, None, None, None) == 0
        assert fn(None, None, None, 0, 100, None, 100, None, None, 0, 24, 2048, f, None, None, None) == 0
        assert fn(None, None, None, 0, 100, None, 100, None, None, 0, 12, 2048, f, None, None, None) == 3
    assert L.dsa_sparse_mla_decode(None, None, None, 0, 100, None, 100, None, None, 0, 128, 2048, f, None, None,
                                   0, None, 0, None) == 0
    assert L.dsa_sparse_mla_decode(None, None, None, 0, 100, None, 100, None, None, 0, 128, 2048, f, None, None,
                                   40, None, 0, None) == 3
