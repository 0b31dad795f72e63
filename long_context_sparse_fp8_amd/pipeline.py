"""One pass of the DSA hot path, as a sequence of C-ABI calls.

prefill_step: cache stores -> indexer scores -> top-k -> sparse MLA (prefill)
decode_step:  cache stores -> indexer scores + top-k (fused) -> sparse MLA (decode)

The caller owns every buffer (`PrefillState` / `DecodeState` hold them so a
timed loop allocates nothing); each stage is one call into libdsa.so on the
current stream.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B


@dataclass
class PrefillState:
    key_cache: torch.Tensor        # [n_pages, 64, d_i] uint8
    key_scale: torch.Tensor        # [n_pages, 64] f32
    kv_cache: torch.Tensor         # [n_slots, 576] bf16, or uint8 for an FP8 cache
    kv_scale: Optional[torch.Tensor]
    scores: torch.Tensor           # [rows, ld] f32
    idx: torch.Tensor              # [rows, k] int32
    out: torch.Tensor              # [rows, H, 512] bf16
    lse: Optional[torch.Tensor]    # [rows, H] f32


def alloc_prefill(n_pages, d_i, n_slots, rows, ld, k, h, kv_fp8=False, with_lse=True, device="cuda"):
    kv_cache = torch.zeros((n_slots, B.DK), dtype=torch.uint8 if kv_fp8 else torch.bfloat16, device=device)
    return PrefillState(
        key_cache=torch.zeros((n_pages, B.PAGE, d_i), dtype=torch.uint8, device=device),
        key_scale=torch.zeros((n_pages, B.PAGE), dtype=torch.float32, device=device),
        kv_cache=kv_cache,
        kv_scale=torch.zeros(n_slots, dtype=torch.float32, device=device) if kv_fp8 else None,
        scores=torch.empty((rows, ld), dtype=torch.float32, device=device),
        idx=torch.empty((rows, k), dtype=torch.int32, device=device),
        out=torch.empty((rows, h, B.DV), dtype=torch.bfloat16, device=device),
        lse=torch.empty((rows, h), dtype=torch.float32, device=device) if with_lse else None,
    )


def store_tokens(st: PrefillState, ik, ik_scale, ik_slot, kv, kv_slot):
    """Write new tokens' indexer keys and latent rows into the two caches (one launch)."""
    B.cache_store(ik, ik_scale, ik_slot, st.key_cache, st.key_scale, kv, kv_slot, st.kv_cache, st.kv_scale)


def prefill_step(st: PrefillState, iq, iq_scale, w, page_table, kv_slot_table, q_seq, q_pos, q, k, sm_scale,
                 row0=0, rows=None):
    """Indexer -> top-k -> sparse MLA for query rows [row0, row0 + rows) of the given
    query tensors (the caches must already hold every key those rows can see)."""
    n = iq.shape[0] if rows is None else rows
    sc = st.scores[:n]
    ix = st.idx[:n]
    B.indexer_scores(iq, iq_scale, w, st.key_cache, st.key_scale, page_table, q_seq, q_pos, sc)
    B.topk(sc, q_pos, k, ix)
    B.sparse_mla_prefill(q, st.kv_cache, kv_slot_table, q_seq, ix, sm_scale, st.out[:n],
                         st.lse[:n] if st.lse is not None else None, kv_scale=st.kv_scale)


@dataclass
class DecodeState:
    scores: torch.Tensor           # [B, ld] f32
    idx: torch.Tensor              # [B, k] int32
    out: torch.Tensor              # [B, H, 512] bf16
    lse: torch.Tensor              # [B, H] f32
    ws: torch.Tensor               # sparse MLA decode workspace (uint8)
    n_splits: int
    topk_ws: Optional[torch.Tensor] = None   # top-k workspace (uint8), None when rows are not split
    fused_ws: Optional[torch.Tensor] = None  # workspace of the fused indexer -> top-k (uint8, zeroed once)


def alloc_decode(batch, ld, k, h, n_splits=0, fused=True, device="cuda"):
    """Buffers of one decode step over contexts of up to `ld` tokens.  The score
    rows are padded to a multiple of 64 columns so every row is 256-byte aligned
    (the top-k then reads them with 16-byte vector loads).  Every workspace is
    allocated here, so a step allocates nothing.  fused (up to 256 queries): the
    indexer and top-k run as one fused call (its workspace is zeroed here once;
    every call leaves it ready for the next); otherwise as two calls, the long
    rows split over several workgroups."""
    need = B.sparse_mla_decode_workspace_size(batch, h, k, n_splits)
    ld = (ld + 63) // 64 * 64
    fused = fused and batch <= B.INDEXER_DECODE_MAX_Q
    tk = 0 if fused else B.topk_workspace_size(batch, ld, k)
    return DecodeState(scores=torch.empty((batch, ld), dtype=torch.float32, device=device),
                       idx=torch.empty((batch, k), dtype=torch.int32, device=device),
                       out=torch.empty((batch, h, B.DV), dtype=torch.bfloat16, device=device),
                       lse=torch.empty((batch, h), dtype=torch.float32, device=device),
                       ws=torch.empty(max(need, 1), dtype=torch.uint8, device=device), n_splits=n_splits,
                       topk_ws=torch.empty(tk, dtype=torch.uint8, device=device) if tk else None,
                       fused_ws=torch.zeros(B.indexer_topk_workspace_size(batch), dtype=torch.uint8, device=device)
                       if fused else None)


def decode_select(ds: DecodeState, caches: PrefillState, iq, iq_scale, w, page_table, q_seq, q_pos, k):
    """Indexer scores and top-k of a decode step (fused when ds holds the histogram workspace)."""
    if ds.fused_ws is not None:
        B.indexer_topk(iq, iq_scale, w, caches.key_cache, caches.key_scale, page_table, q_seq, q_pos, ds.scores, k,
                       ds.idx, ds.fused_ws)
    else:
        B.indexer_scores(iq, iq_scale, w, caches.key_cache, caches.key_scale, page_table, q_seq, q_pos, ds.scores)
        B.topk(ds.scores, q_pos, k, ds.idx, ws=ds.topk_ws)


def decode_step(ds: DecodeState, caches: PrefillState, iq, iq_scale, w, page_table, kv_slot_table, q_seq, q_pos, q,
                k, sm_scale):
    decode_select(ds, caches, iq, iq_scale, w, page_table, q_seq, q_pos, k)
    B.sparse_mla_decode(q, caches.kv_cache, kv_slot_table, q_seq, ds.idx, sm_scale, ds.out, ds.lse,
                        kv_scale=caches.kv_scale, n_splits=ds.n_splits, ws=ds.ws)
