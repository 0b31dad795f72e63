"""The seeded input recipe (no GPU): every tensor is reproducible from its
seed, tensors drawn with more rows extend the smaller draw, and the stated
shapes, distributions and page / slot layouts hold."""
import numpy as np
import torch

import synth
from synth.configs import CONFIGS, PAGE


def _f8(codes):
    return codes.view(torch.float8_e4m3fn).to(torch.float32)


def test_prefill_inputs_are_reproducible_and_nested():
    a = synth.make_prefill("C1")
    b = synth.make_prefill("C1")
    for name in ("iq", "iq_scale", "w", "ik", "ik_scale", "q", "kv", "page_table", "ik_slot", "kv_slot_table"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    c = synth.make_prefill("C1", L=256)         # fewer rows: the leading rows of the same draws
    assert torch.equal(c.kv, a.kv[:256]) and torch.equal(c.q, a.q[:256]) and torch.equal(c.w, a.w[:256])


def test_fp8_per_token_recipe():
    x = synth.normal((64, 16, 64), 1234)
    codes, scale = synth.fp8_per_token(x)
    amax = x.reshape(64, -1).abs().amax(1)
    assert torch.equal(scale, amax / 448.0)
    dec = _f8(codes).reshape(64, -1)
    assert dec.abs().amax(1).eq(448.0).all()                      # each token's largest value lands on 448
    err = (dec * scale[:, None] - x.reshape(64, -1)).abs() / scale[:, None]
    assert err.max() <= 16.0                                      # half an E4M3 step at the top binade (32)
    z, s0 = synth.fp8_per_token(torch.zeros(3, 8))
    assert torch.equal(s0, torch.ones(3)) and z.eq(0).all()


def test_prefill_distributions_and_layout():
    cfg = CONFIGS["C2"]
    inp = synth.make_prefill(cfg, L=2048, materialize_q=False)
    w = inp.w.double()
    assert abs(w.var().item() - 1.0 / cfg.h_i) < 0.05 / cfg.h_i   # N(0, 1/H_I) weights
    kv = inp.kv.double()
    assert abs(kv.mean().item()) < 0.01 and abs(kv.std().item() - 1.0) < 0.01
    assert torch.equal(inp.q_pos, torch.arange(2048, dtype=torch.int32)) and inp.q_seq.eq(0).all()
    # identity layout for C2; seeded permutations for the paged configs
    assert torch.equal(inp.page_table[0], torch.arange(inp.n_pages, dtype=torch.int32))
    p = synth.make_prefill(CONFIGS["C3"], L=4096, materialize_q=False)
    assert torch.equal(p.page_table[0].sort().values, torch.arange(p.n_pages, dtype=torch.int32))
    assert torch.equal(p.kv_slot_table[0].sort().values, torch.arange(4096, dtype=torch.int32))
    s = torch.arange(4096)
    assert torch.equal(p.ik_slot, p.page_table[0].long()[s // PAGE] * PAGE + s % PAGE)


def test_exact_regime_values():
    inp = synth.make_prefill("C1", exact=True)
    for t in (inp.iq, inp.ik):
        v = _f8(t)
        assert v.eq(v.round()).all() and v.abs().max() <= 4
    for s in (inp.iq_scale, inp.ik_scale):
        e = torch.log2(s)
        assert e.eq(e.round()).all() and e.min() >= -3 and e.max() <= 3
    w16 = inp.w * 16
    assert w16.eq(w16.round()).all() and inp.w.abs().max() <= 1


def test_decode_layout():
    d = synth.make_decode("C4", batch=5, ctx_lo=100, ctx_hi=300, queries_per_seq=2)
    lens = d.lens
    assert lens.min() >= 100 and lens.max() <= 300
    assert torch.equal(d.q_pos.long(), (lens.view(-1, 1) - 2 + torch.arange(2).view(1, -1)).reshape(-1))
    assert torch.equal(d.q_seq, torch.arange(5, dtype=torch.int32).repeat_interleave(2))
    used_pages, used_slots = [], []
    for b in range(5):
        n = int(lens[b])
        npg = (n + PAGE - 1) // PAGE
        assert d.page_table[b, :npg].ge(0).all() and d.page_table[b, npg:].eq(-1).all()
        assert d.kv_slot_table[b, :n].ge(0).all() and d.kv_slot_table[b, n:].eq(-1).all()
        used_pages.append(d.page_table[b, :npg])
        used_slots.append(d.kv_slot_table[b, :n])
    # one shuffled pool: every physical page and slot belongs to exactly one sequence
    assert torch.equal(torch.cat(used_pages).sort().values, torch.arange(d.n_pages, dtype=torch.int32))
    assert torch.equal(torch.cat(used_slots).sort().values, torch.arange(int(lens.sum()), dtype=torch.int32))
    one = synth.make_decode("C4", batch=5, ctx_lo=100, ctx_hi=300)
    assert torch.equal(one.lens, lens) and torch.equal(one.q_pos.long(), lens - 1)
