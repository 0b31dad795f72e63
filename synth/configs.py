"""The five DSA workloads as seeded synthetic inputs.

C1  tiny prefill        B=1, L=1024,  k=256,  indexer 16x64,  MLA 8 heads
C2  prefill 8K          B=1, L=8192,  k=2048, indexer 64x128, MLA 128 heads
C3  prefill 32K         B=1, L=32768, k=2048, paged indexer keys (64/page,
                        random page permutation), KV slots randomly permuted
C4  decode              64 sequences, one query each, context ~ U{32768..131072}
                        (inclusive of the query token), scattered pages/slots
C5  chunked prefill     one 131072-token sequence in 8192-token chunks, FP8 KV

Only random draws and storage layouts live here (page tables, the slot each
logical token is stored at); nothing of the method is computed.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

from .gen import (normal, bf16_normal, fp8_per_token, randperm, gen, e1_codes, e1_pow2_scales,
                  e1_weights)

PAGE = 64          # indexer key cache page size (tokens per page)
DK, DV = 576, 512  # latent key width / value width


@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    L: int
    k: int
    h_i: int
    d_i: int
    h: int
    paged: bool = False
    kv_fp8: bool = False
    chunk: int = 0
    decode_batch: int = 0
    ctx_lo: int = 0
    ctx_hi: int = 0


CONFIGS = {
    "C1": Config("C1", 1, L=1024, k=256, h_i=16, d_i=64, h=8),
    "C2": Config("C2", 2, L=8192, k=2048, h_i=64, d_i=128, h=128),
    "C3": Config("C3", 3, L=32768, k=2048, h_i=64, d_i=128, h=128, paged=True),
    "C4": Config("C4", 4, L=0, k=2048, h_i=64, d_i=128, h=128, paged=True,
                 decode_batch=64, ctx_lo=32768, ctx_hi=131072),
    "C5": Config("C5", 5, L=131072, k=2048, h_i=64, d_i=128, h=128, paged=True, kv_fp8=True,
                 chunk=8192),
}

SM_SCALE = 1.0 / 24.0   # 1 / sqrt(576)

# tensor ids (seed = 1000 * cid + id)
T_IQ, T_W, T_IK, T_Q, T_KV, T_PAGE_PERM, T_SLOT_PERM, T_LENS = 1, 3, 4, 5, 6, 7, 8, 9


def _seed(cfg, tid, extra=0):
    return 1000 * cfg.cid + tid + 100000 * extra


@dataclass
class PrefillInputs:
    cfg: Config
    iq: torch.Tensor          # [n_q, H_I, D_I] uint8 E4M3 codes
    iq_scale: torch.Tensor    # [n_q] f32
    w: torch.Tensor           # [n_q, H_I] f32
    ik: torch.Tensor          # [L, D_I] uint8 codes, logical token order
    ik_scale: torch.Tensor    # [L] f32
    q: Optional[torch.Tensor]  # [n_q, H, 576] bf16 (None for chunked: see q_chunk)
    kv: torch.Tensor          # [L, 576] bf16, logical token order
    q_pos: torch.Tensor       # [n_q] int32
    q_seq: torch.Tensor       # [n_q] int32 (all 0)
    page_table: torch.Tensor  # [1, n_pages] int32: logical page -> physical page
    ik_slot: torch.Tensor     # [L] int64: physical page * 64 + offset of each token
    kv_slot_table: torch.Tensor  # [1, L] int32: logical token -> KV slot
    n_pages: int
    n_slots: int
    q_seed: int = 0
    extra: dict = field(default_factory=dict)

    def q_chunk(self, c0, c1):
        """bf16 q rows [c0, c1) (drawn per 8192-row block, so any chunking of
        the same sequence sees the same values)."""
        if self.q is not None:
            return self.q[c0:c1]
        dev = self.kv.device
        blk = 8192
        parts = []
        for b0 in range(c0 - c0 % blk, c1, blk):
            qb = bf16_normal((blk, self.cfg.h, DK), self.q_seed + 7919 * (b0 // blk), dev)
            lo, hi = max(c0, b0) - b0, min(c1, b0 + blk) - b0
            parts.append(qb[lo:hi])
        return torch.cat(parts) if len(parts) > 1 else parts[0]


def _layout(cfg, L, device):
    n_pages = (L + PAGE - 1) // PAGE
    if cfg.paged:
        page_perm = randperm(n_pages, _seed(cfg, T_PAGE_PERM)).to(torch.int32)
        slot_perm = randperm(L, _seed(cfg, T_SLOT_PERM)).to(torch.int32)
    else:
        page_perm = torch.arange(n_pages, dtype=torch.int32)
        slot_perm = torch.arange(L, dtype=torch.int32)
    s = torch.arange(L, dtype=torch.int64)
    ik_slot = page_perm.to(torch.int64)[s // PAGE] * PAGE + s % PAGE
    return (page_perm.reshape(1, -1).to(device), ik_slot.to(device), slot_perm.reshape(1, -1).to(device),
            n_pages, L)


def make_prefill(cfg, device="cpu", exact=False, L=None, materialize_q=True):
    """Inputs of one prefill pass over a single sequence of L tokens.

    exact=True draws the exact-arithmetic set E1 instead of N(0, 1) values
    (indexer only; the MLA tensors stay N(0, 1)).  Large tensors are drawn on
    ``device`` directly."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    L = L or cfg.L
    if exact:
        iq = e1_codes((L, cfg.h_i, cfg.d_i), _seed(cfg, T_IQ, 1)).to(device)
        iq_scale = e1_pow2_scales(L, _seed(cfg, T_IQ, 2)).to(device)
        ik = e1_codes((L, cfg.d_i), _seed(cfg, T_IK, 1)).to(device)
        ik_scale = e1_pow2_scales(L, _seed(cfg, T_IK, 2)).to(device)
        w = e1_weights((L, cfg.h_i), _seed(cfg, T_W, 1)).to(device)
    else:
        iq, iq_scale = fp8_per_token(normal((L, cfg.h_i, cfg.d_i), _seed(cfg, T_IQ), device))
        ik, ik_scale = fp8_per_token(normal((L, cfg.d_i), _seed(cfg, T_IK), device))
        w = normal((L, cfg.h_i), _seed(cfg, T_W), device, std=(1.0 / cfg.h_i) ** 0.5)
    kv = bf16_normal((L, DK), _seed(cfg, T_KV), device)
    q_seed = _seed(cfg, T_Q)
    q = bf16_normal((L, cfg.h, DK), q_seed, device) if materialize_q else None
    page_table, ik_slot, kv_slot_table, n_pages, n_slots = _layout(cfg, L, device)
    return PrefillInputs(cfg=cfg, iq=iq, iq_scale=iq_scale, w=w, ik=ik, ik_scale=ik_scale, q=q, kv=kv,
                         q_pos=torch.arange(L, dtype=torch.int32, device=device),
                         q_seq=torch.zeros(L, dtype=torch.int32, device=device),
                         page_table=page_table, ik_slot=ik_slot, kv_slot_table=kv_slot_table,
                         n_pages=n_pages, n_slots=n_slots, q_seed=q_seed)


@dataclass
class DecodeInputs:
    cfg: Config
    lens: torch.Tensor        # [B] int64 context length of each sequence (incl. the query token)
    seq_start: torch.Tensor   # [B] int64 first logical row of each sequence in ik / kv
    iq: torch.Tensor          # [B m, H_I, D_I] uint8 (m query tokens per sequence, sequence-major)
    iq_scale: torch.Tensor    # [B m]
    w: torch.Tensor           # [B m, H_I]
    ik: torch.Tensor          # [N, D_I] uint8, all sequences concatenated (logical order)
    ik_scale: torch.Tensor    # [N]
    q: torch.Tensor           # [B m, H, 576] bf16
    kv: torch.Tensor          # [N, 576] bf16 (logical order)
    q_pos: torch.Tensor       # [B m] int32: lens - m .. lens - 1 per sequence
    q_seq: torch.Tensor       # [B m] int32: b repeated m times
    page_table: torch.Tensor  # [B, max_pages] int32 (-1 past each sequence's last page)
    ik_slot: torch.Tensor     # [N] int64
    kv_slot_table: torch.Tensor  # [B, max_len] int32 (-1 past each sequence's end)
    n_pages: int
    n_slots: int


def decode_queries(cfg, lens, m=1, device="cpu"):
    """Query-side tensors of a decode step with m query tokens per sequence, at
    the last m positions of each context (the shape multi-token prediction
    presents); m = 1 is the plain one-token step.  Returns (iq, iq_scale, w, q,
    q_pos, q_seq) with rows in sequence-major order."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = lens.numel()
    x = 0 if m == 1 else 10 + m
    iq, iq_scale = fp8_per_token(normal((B * m, cfg.h_i, cfg.d_i), _seed(cfg, T_IQ, x), device))
    w = normal((B * m, cfg.h_i), _seed(cfg, T_W, x), device, std=(1.0 / cfg.h_i) ** 0.5)
    q = bf16_normal((B * m, cfg.h, DK), _seed(cfg, T_Q, x), device)
    q_pos = (lens.cpu().view(-1, 1) - m + torch.arange(m).view(1, -1)).reshape(-1).to(torch.int32)
    q_seq = torch.arange(B, dtype=torch.int32).repeat_interleave(m)
    return iq, iq_scale, w, q, q_pos.to(device), q_seq.to(device)


def make_decode(cfg="C4", device="cpu", batch=None, ctx_lo=None, ctx_hi=None, queries_per_seq=1):
    """One decode step: B sequences, `queries_per_seq` query tokens each at the
    last positions of its context (default one).  Physical pages / slots of all
    sequences are one shuffled pool."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = batch or cfg.decode_batch
    lo, hi = ctx_lo or cfg.ctx_lo, ctx_hi or cfg.ctx_hi
    lens = torch.randint(lo, hi + 1, (B,), generator=gen(_seed(cfg, T_LENS)), dtype=torch.int64)
    N = int(lens.sum())
    seq_start = torch.zeros(B, dtype=torch.int64)
    seq_start[1:] = torch.cumsum(lens, 0)[:-1]
    pages = (lens + PAGE - 1) // PAGE
    n_pages = int(pages.sum())
    max_pages = int(pages.max())
    max_len = int(lens.max())
    page_perm = randperm(n_pages, _seed(cfg, T_PAGE_PERM)).to(torch.int32)
    slot_perm = randperm(N, _seed(cfg, T_SLOT_PERM)).to(torch.int32)
    page_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    kv_slot_table = torch.full((B, max_len), -1, dtype=torch.int32)
    ik_slot = torch.empty(N, dtype=torch.int64)
    p0 = 0
    for b in range(B):
        nb, npg = int(lens[b]), int(pages[b])
        page_table[b, :npg] = page_perm[p0:p0 + npg]
        s = torch.arange(nb, dtype=torch.int64)
        ik_slot[seq_start[b]:seq_start[b] + nb] = page_table[b].to(torch.int64)[s // PAGE] * PAGE + s % PAGE
        kv_slot_table[b, :nb] = slot_perm[seq_start[b]:seq_start[b] + nb]
        p0 += npg
    iq, iq_scale, w, q, q_pos, q_seq = decode_queries(cfg, lens, queries_per_seq, device)
    ik, ik_scale = fp8_per_token(normal((N, cfg.d_i), _seed(cfg, T_IK), device))
    kv = bf16_normal((N, DK), _seed(cfg, T_KV), device)
    return DecodeInputs(cfg=cfg, lens=lens, seq_start=seq_start, iq=iq, iq_scale=iq_scale, w=w, ik=ik,
                        ik_scale=ik_scale, q=q, kv=kv, q_pos=q_pos, q_seq=q_seq,
                        page_table=page_table.to(device), ik_slot=ik_slot.to(device),
                        kv_slot_table=kv_slot_table.to(device), n_pages=n_pages, n_slots=N)
