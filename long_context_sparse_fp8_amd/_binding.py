"""ctypes binding of libdsa.so (the C ABI in include/dsa.h).

Argument marshalling only: each function checks dtypes / shapes / device of
torch tensors, passes raw device pointers plus torch's current HIP stream,
and raises DSAError on a non-OK status.  Every computation runs in the HIP
kernels of the library; there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libdsa.so")

DSA_OK = 0
KV_BF16 = 0
KV_FP8_E4M3 = 1
PAGE = 64
DK = 576
DV = 512
INDEXER_DECODE_MAX_Q = 256   # largest query count of the split-key (decode) scorer and the fused call

_lib = None


class DSAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status}: {message}")
        self.status = status


def lib():
    """Load libdsa.so (built in-tree by long_context_sparse_fp8_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_fp8_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.dsa_abi_version.restype = ctypes.c_int
    L.dsa_abi_version.argtypes = []
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_indexer_cache_store.restype = ctypes.c_int
    L.dsa_indexer_cache_store.argtypes = [P, P, P, i32, i32, P, P, i64, P]
    L.dsa_kv_cache_store.restype = ctypes.c_int
    L.dsa_kv_cache_store.argtypes = [P, P, i32, ctypes.c_int, P, P, i64, P]
    L.dsa_cache_store.restype = ctypes.c_int
    L.dsa_cache_store.argtypes = [P, P, P, i32, i32, P, P, i64, P, P, i32, ctypes.c_int, P, P, i64, P]
    L.dsa_indexer_scores.restype = ctypes.c_int
    L.dsa_indexer_scores.argtypes = [P, P, P, i64, P, P, i64, P, i64, P, P, i32, i32, i32, P, i64, P]
    L.dsa_topk_workspace_size.restype = sz
    L.dsa_topk_workspace_size.argtypes = [i32, i64, i32]
    L.dsa_topk.restype = ctypes.c_int
    L.dsa_topk.argtypes = [P, i64, P, i32, i32, P, P, sz, P]
    L.dsa_indexer_topk_workspace_size.restype = sz
    L.dsa_indexer_topk_workspace_size.argtypes = [i32]
    L.dsa_indexer_topk.restype = ctypes.c_int
    L.dsa_indexer_topk.argtypes = [P, P, P, i64, P, P, i64, P, i64, P, P, i32, i32, i32, P, i64, i32, P, P, sz, P]
    L.dsa_topk_static.restype = ctypes.c_int
    L.dsa_topk_static.argtypes = [P, i64, P, i32, i32, P, P]
    L.dsa_sparse_mla_prefill.restype = ctypes.c_int
    L.dsa_sparse_mla_prefill.argtypes = [P, P, P, ctypes.c_int, i64, P, i64, P, P, i32, i32, i32, f32, P, P, P]
    L.dsa_sparse_mla_decode_workspace_size.restype = sz
    L.dsa_sparse_mla_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    L.dsa_sparse_mla_decode.restype = ctypes.c_int
    L.dsa_sparse_mla_decode.argtypes = [P, P, P, ctypes.c_int, i64, P, i64, P, P, i32, i32, i32, f32, P, P,
                                        i32, P, sz, P]
    _lib = L
    return L


def _check(status):
    if status != DSA_OK:
        L = lib()
        raise DSAError(L.dsa_status_string(status).decode(), L.dsa_last_error().decode())


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def abi_version():
    return lib().dsa_abi_version()


# ---------------------------------------------------------------- cache stores
def indexer_cache_store(k_fp8, k_scale, slot, key_cache, key_scale_cache, stream=None):
    """k_fp8 [n, d_i] uint8; k_scale [n] f32; slot [n] int64 -> key_cache [n_pages, 64, d_i] uint8
    (each page in the fragment-major byte order of dsa.h), key_scale_cache [n_pages, 64] f32 (in place)."""
    n, d_i = k_fp8.shape
    n_pages = key_cache.shape[0]
    assert key_cache.shape[1:] == (PAGE, d_i) and key_scale_cache.shape == (n_pages, PAGE)
    _check(lib().dsa_indexer_cache_store(_ptr(k_fp8, torch.uint8, "k_fp8"), _ptr(k_scale, torch.float32, "k_scale"),
                                         _ptr(slot, torch.int64, "slot"), n, d_i,
                                         _ptr(key_cache, torch.uint8, "key_cache"),
                                         _ptr(key_scale_cache, torch.float32, "key_scale_cache"), n_pages,
                                         _stream(stream)))


def kv_cache_store(kv_bf16, slot, kv_cache, kv_scale=None, stream=None):
    """kv_bf16 [n, 576] bf16; slot [n] int64 -> kv_cache [n_slots, 576] (bf16, or uint8 E4M3 with
    kv_scale [n_slots] f32) in place."""
    n = kv_bf16.shape[0]
    assert kv_bf16.shape[1] == DK and kv_cache.shape[1] == DK
    fp8 = kv_cache.dtype == torch.uint8
    if fp8 and kv_scale is None:
        raise ValueError("kv_scale is required for an FP8 cache")
    _check(lib().dsa_kv_cache_store(_ptr(kv_bf16, torch.bfloat16, "kv_bf16"), _ptr(slot, torch.int64, "slot"), n,
                                    KV_FP8_E4M3 if fp8 else KV_BF16,
                                    _ptr(kv_cache, torch.uint8 if fp8 else torch.bfloat16, "kv_cache"),
                                    _ptr(kv_scale, torch.float32, "kv_scale") if fp8 else None,
                                    kv_cache.shape[0], _stream(stream)))


def cache_store(k_fp8, k_scale, key_slot, key_cache, key_scale_cache, kv_bf16, kv_slot, kv_cache, kv_scale=None,
                stream=None):
    """Both stores in one launch: indexer_cache_store(k_fp8, k_scale, key_slot, key_cache, key_scale_cache)
    and kv_cache_store(kv_bf16, kv_slot, kv_cache, kv_scale), same arguments and results."""
    n_keys, d_i = k_fp8.shape
    n_pages = key_cache.shape[0]
    assert key_cache.shape[1:] == (PAGE, d_i) and key_scale_cache.shape == (n_pages, PAGE)
    n_kv = kv_bf16.shape[0]
    assert kv_bf16.shape[1] == DK and kv_cache.shape[1] == DK
    fp8 = kv_cache.dtype == torch.uint8
    if fp8 and kv_scale is None:
        raise ValueError("kv_scale is required for an FP8 cache")
    _check(lib().dsa_cache_store(_ptr(k_fp8, torch.uint8, "k_fp8"), _ptr(k_scale, torch.float32, "k_scale"),
                                 _ptr(key_slot, torch.int64, "key_slot"), n_keys, d_i,
                                 _ptr(key_cache, torch.uint8, "key_cache"),
                                 _ptr(key_scale_cache, torch.float32, "key_scale_cache"), n_pages,
                                 _ptr(kv_bf16, torch.bfloat16, "kv_bf16"), _ptr(kv_slot, torch.int64, "kv_slot"), n_kv,
                                 KV_FP8_E4M3 if fp8 else KV_BF16,
                                 _ptr(kv_cache, torch.uint8 if fp8 else torch.bfloat16, "kv_cache"),
                                 _ptr(kv_scale, torch.float32, "kv_scale") if fp8 else None,
                                 kv_cache.shape[0], _stream(stream)))


# ---------------------------------------------------------------- stage 1
def indexer_scores(q_fp8, q_scale, w, key_cache, key_scale_cache, page_table, q_seq, q_pos, scores,
                   w_shared=False, stream=None):
    """q_fp8 [n_q, h_i, d_i] uint8; q_scale [n_q]; w [n_q, h_i] (or [h_i] with w_shared);
    key caches as stored; page_table [B, pt_ld] int32; q_seq, q_pos [n_q] int32;
    scores [n_q, ld] f32 (written for columns 0..q_pos)."""
    n_q, h_i, d_i = q_fp8.shape
    _check(lib().dsa_indexer_scores(_ptr(q_fp8, torch.uint8, "q_fp8"), _ptr(q_scale, torch.float32, "q_scale"),
                                    _ptr(w, torch.float32, "w"), 0 if w_shared else h_i,
                                    _ptr(key_cache, torch.uint8, "key_cache"),
                                    _ptr(key_scale_cache, torch.float32, "key_scale_cache"), key_cache.shape[0],
                                    _ptr(page_table, torch.int32, "page_table"), page_table.shape[1],
                                    _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
                                    n_q, h_i, d_i, _ptr(scores, torch.float32, "scores"), scores.shape[1],
                                    _stream(stream)))


# ---------------------------------------------------------------- stage 2
def topk_workspace_size(n_q, max_len, k):
    return int(lib().dsa_topk_workspace_size(n_q, max_len, k))


def topk(scores, q_pos, k, idx, ws=None, stream=None):
    """scores [n_q, ld] f32; q_pos [n_q] int32 -> idx [n_q, k] int32 (ascending, -1 padded)."""
    n_q, ld = scores.shape
    need = topk_workspace_size(n_q, ld, k)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    _check(lib().dsa_topk(_ptr(scores, torch.float32, "scores"), ld, _ptr(q_pos, torch.int32, "q_pos"), n_q, k,
                          _ptr(idx, torch.int32, "idx"), _ptr(ws, None, "ws") if need else None,
                          need, _stream(stream)))


def indexer_topk_workspace_size(n_q):
    return int(lib().dsa_indexer_topk_workspace_size(n_q))


def indexer_topk(q_fp8, q_scale, w, key_cache, key_scale_cache, page_table, q_seq, q_pos, scores, k, idx, ws,
                 w_shared=False, stream=None):
    """indexer_scores then topk with the selection's first pass fused into the scorer (decode form,
    n_q <= 256).  ws: uint8 device tensor of at least indexer_topk_workspace_size(n_q) bytes, zero
    before the first call; every call leaves it ready for the next."""
    n_q, h_i, d_i = q_fp8.shape
    _check(lib().dsa_indexer_topk(_ptr(q_fp8, torch.uint8, "q_fp8"), _ptr(q_scale, torch.float32, "q_scale"),
                                  _ptr(w, torch.float32, "w"), 0 if w_shared else h_i,
                                  _ptr(key_cache, torch.uint8, "key_cache"),
                                  _ptr(key_scale_cache, torch.float32, "key_scale_cache"), key_cache.shape[0],
                                  _ptr(page_table, torch.int32, "page_table"), page_table.shape[1],
                                  _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
                                  n_q, h_i, d_i, _ptr(scores, torch.float32, "scores"), scores.shape[1], k,
                                  _ptr(idx, torch.int32, "idx"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
                                  _stream(stream)))


def topk_static(scores, q_pos, k, idx, stream=None):
    """topk with the library's static workspace (allocates nothing, no workspace argument)."""
    n_q, ld = scores.shape
    _check(lib().dsa_topk_static(_ptr(scores, torch.float32, "scores"), ld, _ptr(q_pos, torch.int32, "q_pos"), n_q,
                                 k, _ptr(idx, torch.int32, "idx"), _stream(stream)))


# ---------------------------------------------------------------- stage 3
def _mla_args(q, kv_cache, kv_scale, kv_slot_table, q_seq, idx, out, lse):
    n_q, h, dk = q.shape
    assert dk == DK and out.shape == (n_q, h, DV) and kv_cache.shape[1] == DK
    fp8 = kv_cache.dtype == torch.uint8
    if fp8 and kv_scale is None:
        raise ValueError("kv_scale is required for an FP8 cache")
    return (_ptr(q, torch.bfloat16, "q"), _ptr(kv_cache, torch.uint8 if fp8 else torch.bfloat16, "kv_cache"),
            _ptr(kv_scale, torch.float32, "kv_scale") if fp8 else None, KV_FP8_E4M3 if fp8 else KV_BF16,
            kv_cache.shape[0], _ptr(kv_slot_table, torch.int32, "kv_slot_table"), kv_slot_table.shape[1],
            _ptr(q_seq, torch.int32, "q_seq"), _ptr(idx, torch.int32, "idx"), n_q, h, idx.shape[1])


def sparse_mla_prefill(q, kv_cache, kv_slot_table, q_seq, idx, sm_scale, out, lse=None, kv_scale=None,
                       stream=None):
    """q [n_q, H, 576] bf16; kv_cache [n_slots, 576] bf16 (or uint8 + kv_scale); kv_slot_table [B, ld]
    int32; q_seq [n_q] int32; idx [n_q, k] int32 -> out [n_q, H, 512] bf16, lse [n_q, H] f32."""
    a = _mla_args(q, kv_cache, kv_scale, kv_slot_table, q_seq, idx, out, lse)
    _check(lib().dsa_sparse_mla_prefill(*a, float(sm_scale), _ptr(out, torch.bfloat16, "out"),
                                        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_mla_decode_workspace_size(n_q, h, k, n_splits=0):
    return int(lib().dsa_sparse_mla_decode_workspace_size(n_q, h, k, n_splits))


def sparse_mla_decode(q, kv_cache, kv_slot_table, q_seq, idx, sm_scale, out, lse=None, kv_scale=None,
                      n_splits=0, ws=None, stream=None):
    """Split-index form of sparse_mla_prefill for few queries; ws is a uint8 device tensor of at
    least sparse_mla_decode_workspace_size(n_q, H, k, n_splits) bytes (allocated here if None)."""
    n_q, h, _ = q.shape
    k = idx.shape[1]
    need = sparse_mla_decode_workspace_size(n_q, h, k, n_splits)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    a = _mla_args(q, kv_cache, kv_scale, kv_slot_table, q_seq, idx, out, lse)
    _check(lib().dsa_sparse_mla_decode(*a, float(sm_scale), _ptr(out, torch.bfloat16, "out"),
                                       _ptr(lse, torch.float32, "lse"), n_splits, _ptr(ws, torch.uint8, "ws"),
                                       ws.numel(), _stream(stream)))
