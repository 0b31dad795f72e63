"""CPU oracle of the DeepSeek Sparse Attention hot path (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and the two share no code.

Thin numpy wrappers around the double-precision C reference in
``dsa_oracle.c`` (see that file for the definitions and their sources):

* ``e4m3_decode`` / ``e4m3_encode`` / ``bf16_decode`` -- number formats
* ``kv_quantize``       -- FP8 latent-row quantization (cache-store reference)
* ``indexer_scores``    -- Lightning Indexer scores (O1)
* ``topk``              -- top-k selection, ascending indices, -1 padded (O2)
* ``sparse_mla``        -- attention over the selected latent rows (O3)
* ``dense_mla``         -- dense causal MLA, every predecessor selected (O4)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

DK = 576   # latent key width (512 value dims + 64 rope dims)
DV = 512


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_decode.restype = ctypes.c_double
    lib.orc_kv_quantize_rows.argtypes = [P, i64, i32, P, P]
    lib.orc_kv_quantize_rows.restype = None
    lib.orc_indexer_scores.argtypes = [i32, i32, i32, P, P, P, i64, P, P, P, P, P, P, i64, i32]
    lib.orc_indexer_scores.restype = i32
    lib.orc_topk.argtypes = [P, i64, P, i32, i32, P, i32]
    lib.orc_topk.restype = i32
    lib.orc_sparse_mla.argtypes = [i32, i32, i32, i32, P, P, P, i32, P, P, P, i32, f32, P, P, i32]
    lib.orc_sparse_mla.restype = i32
    lib.orc_dense_mla.argtypes = [i32, i32, i32, i32, P, P, P, i32, P, P, P, f32, P, P, i32]
    lib.orc_dense_mla.restype = i32
    _lib = lib
    return lib


def _threads(n_threads):
    return int(n_threads) if n_threads else (os.cpu_count() or 1)


def _c(a, dtype):
    a = np.ascontiguousarray(np.asarray(a), dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- formats
def e4m3_decode(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3_decode(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def e4m3_encode(x):
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def bf16_decode(bits):
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.orc_bf16_decode(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def e4m3_table():
    """Exact double value of each of the 256 codes (NaN for the two NaN codes)."""
    return e4m3_decode(np.arange(256, dtype=np.uint8))


# ---------------------------------------------------------------- cache store
def kv_quantize(rows_bf16_bits):
    """[n, w] uint16 bf16 bits -> ([n, w] uint8 E4M3 codes, [n] fp32 scales)."""
    lib = _load()
    rows = _c(rows_bf16_bits, np.uint16)
    n, w = rows.shape
    codes = np.empty((n, w), dtype=np.uint8)
    scales = np.empty((n,), dtype=np.float32)
    lib.orc_kv_quantize_rows(_p(rows), n, w, _p(codes), _p(scales))
    return codes, scales


# ---------------------------------------------------------------- O1
def indexer_scores(q, q_scale, w, k, k_scale, q_pos, *, seq_start=None, q_seq=None,
                   ld=None, w_shared=False, n_threads=None, fill=np.nan):
    """q: [n_q, H_I, D_I] uint8 codes; q_scale [n_q] f32; w [n_q, H_I] f32 (or [H_I]
    with w_shared); k: [N, D_I] uint8 logical key rows; k_scale [N] f32;
    q_pos [n_q]; seq_start [B] int64 (default [0]); q_seq [n_q] (default 0).
    Returns scores [n_q, ld] float32, entries past q_pos set to ``fill``."""
    lib = _load()
    q = _c(q, np.uint8)
    n_q, h_i, d_i = q.shape
    k = _c(k, np.uint8)
    assert k.shape[1] == d_i
    q_scale = _c(q_scale, np.float32)
    w = _c(w, np.float32)
    w_ld = 0 if w_shared else h_i
    q_pos = _c(q_pos, np.int32)
    seq_start = _c(np.zeros(1) if seq_start is None else seq_start, np.int64)
    q_seq = _c(np.zeros(n_q) if q_seq is None else q_seq, np.int32)
    if ld is None:
        ld = int(q_pos.max()) + 1 if n_q else 1
    scores = np.full((n_q, ld), fill, dtype=np.float32)
    rc = lib.orc_indexer_scores(n_q, h_i, d_i, _p(q), _p(q_scale), _p(w), w_ld, _p(k),
                                _p(_c(k_scale, np.float32)), _p(seq_start), _p(q_seq), _p(q_pos),
                                _p(scores), ld, _threads(n_threads))
    assert rc == 0, rc
    return scores


# ---------------------------------------------------------------- O2
def topk(scores, q_pos, k, *, n_threads=None):
    """scores [n_q, ld] float32 -> idx [n_q, k] int32 (ascending, -1 padded)."""
    lib = _load()
    scores = _c(scores, np.float32)
    n_q, ld = scores.shape
    q_pos = _c(q_pos, np.int32)
    idx = np.empty((n_q, k), dtype=np.int32)
    rc = lib.orc_topk(_p(scores), ld, _p(q_pos), n_q, k, _p(idx), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle top-k: NaN score in a candidate range")
    return idx


# ---------------------------------------------------------------- O3 / O4
def _kv_args(kv, kv_scale):
    if kv_scale is None:
        kv = _c(kv, np.uint16)
        return kv, None, 0
    return _c(kv, np.uint8), _c(kv_scale, np.float32), 1


def sparse_mla(q, kv, idx, sm_scale, *, kv_scale=None, seq_start=None, q_seq=None,
               dv=DV, n_threads=None):
    """q [n_q, H, DK] uint16 bf16 bits; kv [N, DK] uint16 bf16 bits, or uint8
    E4M3 codes with kv_scale [N] f32; idx [n_q, k] int32.  Returns (out
    [n_q, H, dv] float64, lse [n_q, H] float64)."""
    lib = _load()
    q = _c(q, np.uint16)
    n_q, h, dk = q.shape
    kv, kvs, fp8 = _kv_args(kv, kv_scale)
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    seq_start = _c(np.zeros(1) if seq_start is None else seq_start, np.int64)
    q_seq = _c(np.zeros(n_q) if q_seq is None else q_seq, np.int32)
    out = np.zeros((n_q, h, dv), dtype=np.float64)
    lse = np.zeros((n_q, h), dtype=np.float64)
    rc = lib.orc_sparse_mla(n_q, h, dk, dv, _p(q), _p(kv), None if kvs is None else _p(kvs), fp8,
                            _p(seq_start), _p(q_seq), _p(idx), k, float(sm_scale), _p(out), _p(lse),
                            _threads(n_threads))
    assert rc == 0, rc
    return out, lse


def dense_mla(q, kv, q_pos, sm_scale, *, kv_scale=None, seq_start=None, q_seq=None,
              dv=DV, n_threads=None):
    lib = _load()
    q = _c(q, np.uint16)
    n_q, h, dk = q.shape
    kv, kvs, fp8 = _kv_args(kv, kv_scale)
    q_pos = _c(q_pos, np.int32)
    seq_start = _c(np.zeros(1) if seq_start is None else seq_start, np.int64)
    q_seq = _c(np.zeros(n_q) if q_seq is None else q_seq, np.int32)
    out = np.zeros((n_q, h, dv), dtype=np.float64)
    lse = np.zeros((n_q, h), dtype=np.float64)
    rc = lib.orc_dense_mla(n_q, h, dk, dv, _p(q), _p(kv), None if kvs is None else _p(kvs), fp8,
                           _p(seq_start), _p(q_seq), _p(q_pos), float(sm_scale), _p(out), _p(lse),
                           _threads(n_threads))
    assert rc == 0, rc
    return out, lse
