"""Pins of the oracle's sparse / dense MLA (O3 / O4).

Checked against torch's scaled_dot_product_attention in float64 on the CPU
(dense causal case, one latent row shared by every head as key, its first
512 dims as value), a pure-Python softmax on a tiny case, the one-index case
(output = that value row exactly) and the dense degeneration of the whole
oracle chain when k covers every predecessor.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth

SM = 1.0 / 24.0
SM32 = float(np.float32(SM))   # the scale argument is an fp32 value


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _sdpa_dense(q, kv_f64, pos, sm):
    """q [n,H,576] f64, kv [N,576] f64 -> out [n,H,512], lse [n,H] (torch float64 SDPA + logsumexp)."""
    n, H, _ = q.shape
    N = kv_f64.shape[0]
    mask = torch.arange(N)[None, :] <= torch.as_tensor(pos)[:, None]          # [n, N]
    qh = q.permute(1, 0, 2)                                                     # [H, n, 576]
    K = kv_f64.unsqueeze(0).expand(H, N, 576)
    V = kv_f64[:, :512].unsqueeze(0).expand(H, N, 512)
    out = F.scaled_dot_product_attention(qh, K, V, attn_mask=mask.unsqueeze(0), scale=sm)
    logits = (qh @ K.transpose(1, 2)) * sm
    lse = torch.logsumexp(logits.masked_fill(~mask.unsqueeze(0), -math.inf), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.T.numpy()


def test_dense_matches_torch_sdpa(orc):
    L, H = 96, 4
    q = synth.bf16_normal((L, H, 576), 31)
    kv = synth.bf16_normal((L, 576), 32)
    pos = np.arange(L, dtype=np.int32)
    out, lse = orc.dense_mla(_bits(q), _bits(kv), pos, SM)
    ref, ref_lse = _sdpa_dense(q.double(), kv.double(), pos, SM32)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_fp8_kv_matches_torch_sdpa(orc):
    L, H = 64, 2
    q = synth.bf16_normal((L, H, 576), 33)
    kv = synth.bf16_normal((L, 576), 34)
    codes, scales = orc.kv_quantize(_bits(kv))
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).double() * torch.from_numpy(scales).double()[:, None]
    pos = np.arange(L, dtype=np.int32)
    out, lse = orc.dense_mla(_bits(q), codes, pos, SM, kv_scale=scales)
    ref, ref_lse = _sdpa_dense(q.double(), deq, pos, SM32)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_sparse_pure_python_tiny(orc):
    rng = np.random.default_rng(8)
    n, H, N, k = 3, 2, 12, 5
    q = synth.bf16_normal((n, H, 576), 35)
    kv = synth.bf16_normal((N, 576), 36)
    idx = np.full((n, k), -1, np.int32)
    for t in range(n):
        sel = np.sort(rng.choice(N, size=k - t, replace=False))
        idx[t, :len(sel)] = sel
    out, lse = orc.sparse_mla(_bits(q), _bits(kv), idx, SM)
    qd, kd = q.double().numpy().tolist(), kv.double().numpy().tolist()
    for t in range(n):
        S = [int(s) for s in idx[t] if s >= 0]
        for h in range(H):
            ls = [SM32 * sum(a * b for a, b in zip(qd[t][h], kd[s])) for s in S]
            m = max(ls)
            ps = [math.exp(x - m) for x in ls]
            z = sum(ps)
            o = [sum(p * kd[s][d] for p, s in zip(ps, S)) / z for d in range(512)]
            np.testing.assert_allclose(out[t, h], o, rtol=0, atol=1e-12)
            assert abs(lse[t, h] - (m + math.log(z))) < 1e-12


def test_single_index_returns_value_row(orc):
    n, H, N = 4, 3, 10
    q = synth.bf16_normal((n, H, 576), 37)
    kv = synth.bf16_normal((N, 576), 38)
    idx = np.full((n, 6), -1, np.int32)
    idx[:, 0] = [0, 9, 4, 4]
    out, lse = orc.sparse_mla(_bits(q), _bits(kv), idx, SM)
    kvd = kv.double().numpy()
    for t in range(n):
        for h in range(H):
            np.testing.assert_array_equal(out[t, h], kvd[idx[t, 0], :512])
            assert lse[t, h] == pytest.approx(SM32 * float(q[t, h].double() @ kv[idx[t, 0]].double()), abs=1e-12)


def test_empty_selection(orc):
    q = synth.bf16_normal((1, 2, 576), 39)
    kv = synth.bf16_normal((4, 576), 40)
    out, lse = orc.sparse_mla(_bits(q), _bits(kv), np.full((1, 3), -1, np.int32), SM)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_chain_with_k_covering_all_is_dense(orc):
    """Indexer -> top-k (k >= L) -> sparse MLA equals dense causal MLA."""
    inp = synth.make_prefill("C1", L=128)
    iq, ik = inp.iq.numpy(), inp.ik.numpy()
    pos = inp.q_pos.numpy()
    s = orc.indexer_scores(iq, inp.iq_scale.numpy(), inp.w.numpy(), ik, inp.ik_scale.numpy(), pos)
    idx = orc.topk(s, pos, 128)
    out, lse = orc.sparse_mla(_bits(inp.q), _bits(inp.kv), idx, SM)
    dout, dlse = orc.dense_mla(_bits(inp.q), _bits(inp.kv), pos, SM)
    np.testing.assert_array_equal(out, dout)
    np.testing.assert_array_equal(lse, dlse)


def test_multi_sequence_rows(orc):
    """Rows of one sequence in a concatenated KV array: seq_start offsets."""
    H = 2
    kv = synth.bf16_normal((30, 576), 41)
    q = synth.bf16_normal((2, H, 576), 42)
    idx = np.array([[0, 3, 7], [1, 2, -1]], np.int32)
    both, lb = orc.sparse_mla(_bits(q), _bits(kv), idx, SM, seq_start=np.int64([0, 10]), q_seq=np.int32([0, 1]))
    a, _ = orc.sparse_mla(_bits(q[:1]), _bits(kv[:10]), idx[:1], SM)
    b, _ = orc.sparse_mla(_bits(q[1:]), _bits(kv[10:]), idx[1:], SM)
    np.testing.assert_array_equal(both[0], a[0])
    np.testing.assert_array_equal(both[1], b[0])
