"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
(long_context_sparse_fp8_amd) and the CPU oracle on the same seeded inputs."""
import sys
import time

import numpy as np
import torch

import oracle
import synth
from synth.configs import SM_SCALE
import long_context_sparse_fp8_amd as dsa
from long_context_sparse_fp8_amd import pipeline as P

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint8)


def key_cache_rows(key_cache, d_i):
    """[n_pages, 64, d_i] uint8 key cache in the stored fragment-major page order
    -> [n_pages * 64, d_i] rows (key s of page p at row 64 p + s).  Each page is
    a run of 1 KB blocks; block (kt * d_i / 64 + c) * 2 + h, 16-byte slot l holds
    bytes 32 c + 16 h .. +16 of the half g = l // 32 of key 32 kt + l % 32."""
    pages = u8(key_cache).reshape(-1, 64 * d_i)
    half = d_i // 2
    out = np.empty((pages.shape[0], 64, d_i), np.uint8)
    for kt in range(2):
        for c in range(d_i // 64):
            for h in range(2):
                blk = (kt * (d_i // 64) + c) * 2 + h
                for l in range(64):
                    g, key = l // 32, 32 * kt + l % 32
                    b0 = g * half + 32 * c + 16 * h
                    out[:, key, b0:b0 + 16] = pages[:, blk * 1024 + 16 * l:blk * 1024 + 16 * l + 16]
    return out.reshape(-1, d_i)


def max_abs_rel(gpu, ref):
    ref = np.asarray(ref, np.float64)
    gpu = np.asarray(gpu, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / den) if den > 0 else float(np.abs(gpu).max())


def indexer_abs_scale(iq, iq_scale, w, ik, ik_scale, rows, seq_start=0):
    """A[t, s] = qs_t ks_s sum_j |w_tj| sum_i |q_tji k_si| for the given rows (float64):
    the magnitude the FP8 MFMA rounding error is measured against."""
    qv = np.abs(torch.from_numpy(u8(iq[rows]).copy()).view(torch.float8_e4m3fn).double().numpy())  # [r, H, D]
    kv = np.abs(torch.from_numpy(u8(ik).copy()).view(torch.float8_e4m3fn).double().numpy())       # [N, D]
    wa = np.abs(w[rows].double().cpu().numpy())                                                       # [r, H]
    v = np.einsum("rh,rhd->rd", wa, qv)
    A = (v @ kv.T) * iq_scale[rows].double().cpu().numpy()[:, None] * ik_scale.double().cpu().numpy()[None, :]
    return A


def setup_prefill(inp, k, kv_fp8=False, ld=None):
    """Caches filled through the library's cache-store calls; buffers for all rows."""
    cfg = inp.cfg
    L = inp.iq.shape[0]
    ld = ld or L
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, L, ld, k, cfg.h, kv_fp8=kv_fp8)
    P.store_tokens(st, inp.ik.to(DEV), inp.ik_scale.to(DEV), inp.ik_slot.to(DEV), inp.kv.to(DEV),
                   inp.kv_slot_table[0].to(DEV).long())
    return st


def run_prefill(inp, k, kv_fp8=False, rows=None):
    st = setup_prefill(inp, k, kv_fp8)
    d = lambda x: x.to(DEV)
    q = inp.q if inp.q is not None else inp.q_chunk(0, inp.iq.shape[0])
    P.prefill_step(st, d(inp.iq), d(inp.iq_scale), d(inp.w), d(inp.page_table), d(inp.kv_slot_table),
                   d(inp.q_seq), d(inp.q_pos), d(q), k, SM_SCALE)
    torch.cuda.synchronize()
    return st


def oracle_threads():
    import os
    return min(16, os.cpu_count() or 1)
