"""GPU parity of the HIP path (called through the C ABI) against the CPU oracle,
at sizes the oracle finishes in seconds: the tiny prefill (L=1024, 16x64
indexer, 8 MLA heads, k=256) in full, the 64x128 / 128-head shapes on
shortened sequences, ragged tails and the edge cases of the method.

Index parity follows three levels (the GPU's FP8 MFMA sums in an order and
precision of its own, so its fp32 scores can differ from the exact oracle in
the last bits):
  1. top-k from identical scores is bit-exact, always;
  2. in the exact-arithmetic regime E1 every evaluation order gives the same
     bits, so scores and the indexer -> top-k indices are bit-exact end to end;
  3. on N(0, 1) inputs every GPU score is within an a-priori bound of the
     exact score (and the 5e-2 FP8 tolerance).
Sparse-MLA outputs are compared with the oracle evaluated on the GPU's own
indices: max-abs relative error <= 2e-2 (bf16 KV) and 5e-2 (FP8 KV).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import CONFIGS, SM_SCALE, Config
from gpu_common import (DEV, say, bits16, u8, max_abs_rel, indexer_abs_scale, setup_prefill, run_prefill,
                        oracle_threads, key_cache_rows)
import long_context_sparse_fp8_amd as dsa
from long_context_sparse_fp8_amd import pipeline as P

pytestmark = pytest.mark.gpu

# |gpu - exact| <= 2^-15 * sum of |terms|: the FP8 MFMA's measured error bound on
# N(0, 1) inputs quantized per token (test_gpu_numerics.py measures it, with
# adversarial inputs held to the 2^-11 worst case of the MFMA's summation)
BOUND_C = 2.0 ** -15
TOL_BF16, TOL_FP8 = 2e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dsa.lib()


def _cfg(base, **kw):
    d = dict(CONFIGS[base].__dict__)
    d.update(kw)
    return Config(**d)


# ------------------------------------------------------------------ cache stores
@pytest.mark.parametrize("cfg", ["C1", "C3"])
def test_cache_store_bytes(cfg):
    say(f"[cache_store] {cfg}")
    c = _cfg(cfg, L=2048) if cfg == "C3" else CONFIGS[cfg]
    inp = synth.make_prefill(c, L=c.L, materialize_q=False)
    st = setup_prefill(inp, c.k)
    torch.cuda.synchronize()
    slots = inp.ik_slot.numpy()
    kc = key_cache_rows(st.key_cache, c.d_i)
    np.testing.assert_array_equal(kc[slots], u8(inp.ik))
    np.testing.assert_array_equal(st.key_scale.cpu().numpy().reshape(-1)[slots], inp.ik_scale.numpy())
    kvs = inp.kv_slot_table[0].numpy()
    np.testing.assert_array_equal(bits16(st.kv_cache)[kvs], bits16(inp.kv))


def test_cache_stores_skip_out_of_range_slots():
    """Tokens whose slot is negative or past the cache are skipped; every other
    token lands where its slot says, and nothing else in the caches changes."""
    say("[cache_store] out-of-range slots")
    n, n_pages, d_i = 40, 2, 128
    g = synth.gen(4242)
    ik = torch.randint(0, 256, (n, d_i), generator=g, dtype=torch.int64).to(torch.uint8)
    ik[ik == 0x7F] = 0
    iks = torch.rand(n, generator=g) + 0.5
    kv = synth.bf16_normal((n, 576), 4243)
    slot = torch.arange(n, dtype=torch.int64) * 3
    slot[[1, 7]] = -1
    slot[[2, 9]] = n_pages * 64 + torch.tensor([0, 5])           # past the indexer cache
    key_cache = torch.full((n_pages, 64, d_i), 0x11, dtype=torch.uint8, device=DEV)
    key_scale = torch.full((n_pages, 64), -3.0, device=DEV)
    dsa.indexer_cache_store(ik.to(DEV), iks.to(DEV), slot.to(DEV), key_cache, key_scale)
    n_slots = 100
    kv_slot = slot.clone()
    kv_slot[kv_slot >= n_slots] = n_slots + 1                     # past the KV cache too
    kv_cache = torch.full((n_slots, 576), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dsa.kv_cache_store(kv.to(DEV), kv_slot.to(DEV), kv_cache)
    torch.cuda.synchronize()
    rows = key_cache_rows(key_cache, d_i)
    sc = key_scale.cpu().numpy().reshape(-1)
    kvc = bits16(kv_cache.cpu())
    want_rows = np.full((n_pages * 64, d_i), 0x11, np.uint8)
    want_sc = np.full(n_pages * 64, -3.0, np.float32)
    want_kv = np.full((n_slots, 576), 0x1234, np.uint16)
    for i in range(n):
        sl = int(slot[i])
        if 0 <= sl < n_pages * 64:
            want_rows[sl] = u8(ik[i])
            want_sc[sl] = float(iks[i])
        if 0 <= int(kv_slot[i]) < n_slots:
            want_kv[int(kv_slot[i])] = bits16(kv[i])
    np.testing.assert_array_equal(rows, want_rows)
    np.testing.assert_array_equal(sc, want_sc)
    np.testing.assert_array_equal(kvc, want_kv)


def test_cache_store_fp8_matches_oracle_quantizer():
    say("[cache_store] fp8 kv")
    n, n_slots = 777, 1000
    kv = synth.bf16_normal((n, 576), 901)
    kv[3] = 0.0                                          # all-zero row -> scale 1
    kv[5, :7] = torch.tensor([1e-8, -3e-7, 2.0 ** -133, 5e4, -5e4, 0.0, 1.0], dtype=torch.bfloat16)
    slot = synth.randperm(n_slots, 902)[:n].long()
    slot[10] = -1                                        # skipped
    cache = torch.zeros((n_slots, 576), dtype=torch.uint8, device=DEV)
    scale = torch.full((n_slots,), -1.0, dtype=torch.float32, device=DEV)
    dsa.kv_cache_store(kv.to(DEV), slot.to(DEV), cache, scale)
    torch.cuda.synchronize()
    codes, scales = oracle.kv_quantize(bits16(kv))
    s = slot.numpy()
    ok = s >= 0
    np.testing.assert_array_equal(u8(cache)[s[ok]], codes[ok])
    np.testing.assert_array_equal(scale.cpu().numpy()[s[ok]], scales[ok])
    assert scale.cpu().numpy()[np.setdiff1d(np.arange(n_slots), s[ok])].max() == -1.0


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_cache_store_one_launch_equals_the_two_stores(kv_fp8):
    """dsa_cache_store writes the bytes the two separate stores write (different
    key and row counts, slots past either cache and negative slots skipped), a
    zero count leaves that cache untouched, and both zero change nothing."""
    say(f"[cache_store] one launch, fp8={kv_fp8}")
    n_keys, n_kv, n_pages, d_i, n_slots = 70, 45, 2, 128, 90
    g = synth.gen(4343)
    ik = torch.randint(0, 256, (n_keys, d_i), generator=g, dtype=torch.int64).to(torch.uint8)
    iks = torch.rand(n_keys, generator=g) + 0.5
    key_slot = synth.randperm(n_pages * 64 + 12, 4344)[:n_keys].long()     # some past the key cache
    key_slot[3] = -1
    kv = synth.bf16_normal((n_kv, 576), 4345)
    kv_slot = synth.randperm(n_slots + 6, 4346)[:n_kv].long()               # some past the latent cache
    kv_slot[4] = -1
    d = lambda x: x.to(DEV)

    def fresh():
        kc = torch.full((n_pages, 64, d_i), 0x11, dtype=torch.uint8, device=DEV)
        ks = torch.full((n_pages, 64), -3.0, device=DEV)
        if kv_fp8:
            return [kc, ks, torch.full((n_slots, 576), 0x22, dtype=torch.uint8, device=DEV),
                    torch.full((n_slots,), -1.0, device=DEV)]
        return [kc, ks, torch.full((n_slots, 576), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16), None]

    raw = lambda t: t.cpu().contiguous().view(torch.uint8)
    two, one, keys_only, rows_only, none, untouched = (fresh() for _ in range(6))
    dsa.indexer_cache_store(d(ik), d(iks), d(key_slot), two[0], two[1])
    dsa.kv_cache_store(d(kv), d(kv_slot), two[2], two[3])
    dsa.cache_store(d(ik), d(iks), d(key_slot), one[0], one[1], d(kv), d(kv_slot), one[2], one[3])
    dsa.cache_store(d(ik), d(iks), d(key_slot), keys_only[0], keys_only[1], d(kv[:0]), d(kv_slot[:0]),
                    keys_only[2], keys_only[3])
    dsa.cache_store(d(ik[:0]), d(iks[:0]), d(key_slot[:0]), rows_only[0], rows_only[1], d(kv), d(kv_slot),
                    rows_only[2], rows_only[3])
    dsa.cache_store(d(ik[:0]), d(iks[:0]), d(key_slot[:0]), none[0], none[1], d(kv[:0]), d(kv_slot[:0]),
                    none[2], none[3])
    torch.cuda.synchronize()
    n_parts = 4 if kv_fp8 else 3
    for i in range(n_parts):
        assert torch.equal(raw(one[i]), raw(two[i])), i
        assert torch.equal(raw(none[i]), raw(untouched[i])), i
        assert torch.equal(raw(keys_only[i]), raw(two[i] if i < 2 else untouched[i])), i
        assert torch.equal(raw(rows_only[i]), raw(untouched[i] if i < 2 else two[i])), i
    assert not torch.equal(raw(two[0]), raw(untouched[0])) and not torch.equal(raw(two[2]), raw(untouched[2]))


# ------------------------------------------------------------------ indexer
def _oracle_scores(inp, rows, ld):
    return oracle.indexer_scores(u8(inp.iq[rows]), inp.iq_scale[rows].numpy(), inp.w[rows].numpy(), u8(inp.ik),
                                 inp.ik_scale.numpy(), inp.q_pos[rows].numpy(), ld=ld, n_threads=oracle_threads())


@pytest.mark.parametrize("base,L,paged", [("C1", 1024, False), ("C1", 1000, True), ("C2", 2048, False),
                                          ("C3", 2560, True), ("C2", 200, True)])
def test_indexer_exact_regime_bitexact(base, L, paged):
    """E1: integer FP8 codes, power-of-two scales, weights in (1/16)Z: the GPU
    scores equal the oracle's bit for bit, and so do the selected indices."""
    say(f"[indexer E1] {base} L={L} paged={paged}")
    c = _cfg(base, paged=paged)
    inp = synth.make_prefill(c, exact=True, L=L)
    st = run_prefill(inp, c.k)
    g = st.scores.cpu().numpy()
    rows = np.arange(L)
    ref = _oracle_scores(inp, rows, L)
    mask = np.arange(L)[None, :] <= inp.q_pos.numpy()[:, None]
    assert np.array_equal(g[mask], ref[mask]), f"{(g[mask] != ref[mask]).sum()} score mismatches"
    ridx = oracle.topk(ref, inp.q_pos.numpy(), c.k, n_threads=oracle_threads())
    np.testing.assert_array_equal(st.idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("base,L,paged", [("C1", 1024, False), ("C2", 1536, True), ("C2", 777, False)])
def test_indexer_normal_within_bound(base, L, paged):
    say(f"[indexer N(0,1)] {base} L={L} paged={paged}")
    c = _cfg(base, paged=paged)
    inp = synth.make_prefill(c, L=L)
    st = run_prefill(inp, c.k)
    g = st.scores.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, L, max(1, L // 97)), np.arange(max(0, L - 9), L)]))
    ref = _oracle_scores(inp, rows, L)
    A = indexer_abs_scale(inp.iq, inp.iq_scale, inp.w, inp.ik, inp.ik_scale, rows)
    mask = np.arange(L)[None, :] <= inp.q_pos.numpy()[rows][:, None]
    err = np.abs(g[rows] - ref)[mask]
    bound = BOUND_C * A[mask] + 1e-30
    ratio = float((err / bound).max())
    say(f"  max |gpu-exact| / (2^-15 * sum|terms|) = {ratio:.4f}; max-abs-rel = {max_abs_rel(g[rows][mask], ref[mask]):.2e}")
    assert ratio <= 1.0
    assert max_abs_rel(g[rows][mask], ref[mask]) <= TOL_FP8


@pytest.mark.parametrize("n_q,side", [(2, "q"), (300, "q"), (2, "k"), (300, "k")])
def test_indexer_every_code_exact(n_q, side):
    """side q: keys one-hot at 1.0, so score[t, s] = ReLU(q[t, 0, s]); side k: query
    head 0 one-hot at dim t % 128, so score[t, s] = ReLU(k[s, t % 128]).  Unit
    scales and weight: every finite E4M3 code (subnormals, +-0, +-448) on either
    MFMA operand goes through the scorer, the ReLU and the weighting bit-exactly,
    in both scorers (n_q = 2: split-key; 300: query-blocked), with 128 keys over
    two shuffled pages of the fragment-major cache."""
    say(f"[indexer] every code on {side}, n_q={n_q}")
    H, D, N = 64, 128, 128
    codes = np.arange(256, dtype=np.int64)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]                         # 254 finite codes
    q = np.zeros((n_q, H, D), np.uint8)
    k = np.zeros((N, D), np.uint8)
    if side == "q":
        for t in range(n_q):
            q[t, 0] = np.roll(codes, -37 * t)[:D] if t % 2 == 0 else np.roll(codes, -37 * t)[D - 2:2 * D - 2]
        k[np.arange(N), np.arange(N)] = 0x38                                    # E4M3 1.0
    else:
        q[np.arange(n_q), 0, np.arange(n_q) % D] = 0x38
        for s_ in range(N):
            k[s_] = np.roll(codes, -29 * s_)[:D] if s_ % 2 == 0 else np.roll(codes, -29 * s_)[D - 2:2 * D - 2]
    w = np.zeros((n_q, H), np.float32)
    w[:, 0] = 1.0
    page_of = np.array([1, 0])                                                  # logical page -> physical
    slot = torch.tensor(page_of[np.arange(N) // 64] * 64 + np.arange(N) % 64, dtype=torch.int64, device=DEV)
    key_cache = torch.zeros((2, 64, D), dtype=torch.uint8, device=DEV)
    key_scale = torch.zeros((2, 64), dtype=torch.float32, device=DEV)
    dsa.indexer_cache_store(torch.from_numpy(k).to(DEV), torch.ones(N, device=DEV), slot, key_cache, key_scale)
    scores = torch.full((n_q, N), -5.0, device=DEV)
    dsa.indexer_scores(torch.from_numpy(q).to(DEV), torch.ones(n_q, device=DEV), torch.from_numpy(w).to(DEV),
                       key_cache, key_scale, torch.tensor(page_of, dtype=torch.int32, device=DEV).reshape(1, 2),
                       torch.zeros(n_q, dtype=torch.int32, device=DEV),
                       torch.full((n_q,), N - 1, dtype=torch.int32, device=DEV), scores)
    torch.cuda.synchronize()
    if side == "q":
        val = torch.from_numpy(q[:, 0, :].copy()).view(torch.float8_e4m3fn).float().numpy()
    else:
        kv_ = torch.from_numpy(k.copy()).view(torch.float8_e4m3fn).float().numpy()
        val = kv_[:, np.arange(n_q) % D].T                                     # [n_q, N]
    want = np.maximum(val, 0.0) + 0.0                                           # +0 for every non-positive code
    np.testing.assert_array_equal(scores.cpu().numpy().view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_indexer_decode_pages_past_the_table_give_nan():
    """Split-key scorer, rows longer than 64 pages of a short page table: every
    logical page from pt_ld up to the row's position gets NaN scores (the
    workgroups cover the score row, not just the table), the table's pages keep
    their scores, and columns past the position stay untouched."""
    say("[indexer] decode rows reaching past the page table")
    c = _cfg("C2", paged=True)
    L, n_q, pt_ld = 5000, 2, 10
    inp = synth.make_prefill(c, L=L, materialize_q=False)
    st = setup_prefill(inp, c.k)
    d = lambda x: x.to(DEV)
    rows = np.array([640, 4500])                                # one query per sequence, positions >= 4160
    table = d(inp.page_table[:, :pt_ld]).contiguous().expand(2, pt_ld).contiguous()
    pos = torch.tensor([4200, 4999], dtype=torch.int32)
    sc = torch.full((n_q, L), -7.0, device=DEV)
    dsa.indexer_scores(d(inp.iq[rows]), d(inp.iq_scale[rows]), d(inp.w[rows]), st.key_cache, st.key_scale,
                       table, torch.arange(n_q, dtype=torch.int32, device=DEV), d(pos), sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    ref = oracle.indexer_scores(u8(inp.iq[rows]), inp.iq_scale[rows].numpy(), inp.w[rows].numpy(), u8(inp.ik),
                                inp.ik_scale.numpy(), np.full(n_q, 64 * pt_ld - 1, np.int32), ld=64 * pt_ld)
    A = indexer_abs_scale(inp.iq, inp.iq_scale, inp.w, inp.ik, inp.ik_scale, rows)[:, :64 * pt_ld]
    for r in range(n_q):
        p = int(pos[r])
        assert (np.abs(got[r, :64 * pt_ld] - ref[r]) <= BOUND_C * A[r] + 1e-30).all(), r
        assert np.isnan(got[r, 64 * pt_ld:p + 1]).all(), r
        assert (got[r, p + 1:] == -7.0).all(), r


@pytest.mark.parametrize("n_q", [4, 300])
def test_indexer_absent_pages_give_nan(n_q):
    """A page-table entry of -1, one past n_pages, and a logical page past pt_ld
    give NaN scores for exactly their 64 tokens; every other score equals the
    complete table's bit for bit (both scorers)."""
    say(f"[indexer] absent pages, n_q={n_q}")
    c = _cfg("C2", paged=True)
    L = 700
    inp = synth.make_prefill(c, L=L, materialize_q=False)
    st = setup_prefill(inp, c.k)
    rows = np.arange(L - n_q, L)
    d = lambda x: x.to(DEV)
    def scores(table):
        sc = torch.full((n_q, L), -7.0, device=DEV)
        dsa.indexer_scores(d(inp.iq[rows]), d(inp.iq_scale[rows]), d(inp.w[rows]), st.key_cache, st.key_scale,
                           table, torch.zeros(n_q, dtype=torch.int32, device=DEV),
                           d(inp.q_pos[rows]).contiguous(), sc)
        torch.cuda.synchronize()
        return sc.cpu().numpy()
    full = scores(d(inp.page_table).contiguous())
    bad = inp.page_table.clone()[:, :10].contiguous()          # logical page 10 is past pt_ld
    bad[0, 3] = -1
    bad[0, 5] = inp.n_pages + 7
    got = scores(d(bad))
    pos = inp.q_pos[rows].numpy()
    page = np.arange(L) // 64
    for r in range(n_q):
        valid = np.arange(L) <= pos[r]
        gone = valid & np.isin(page, [3, 5, 10])
        assert np.isnan(got[r, gone]).all(), r
        keep = valid & ~gone
        np.testing.assert_array_equal(got[r, keep].view(np.uint32), full[r, keep].view(np.uint32))
        assert (got[r, ~valid] == -7.0).all()                  # columns past q_pos untouched


def test_indexer_shared_weights_and_columns_untouched():
    say("[indexer] shared weights, untouched columns")
    c = CONFIGS["C1"]
    inp = synth.make_prefill(c, L=300)
    st = setup_prefill(inp, c.k, ld=320)
    st.scores.fill_(12345.0)
    w0 = inp.w[0].contiguous()
    dsa.indexer_scores(inp.iq.to(DEV), inp.iq_scale.to(DEV), w0.to(DEV), st.key_cache, st.key_scale,
                       inp.page_table.to(DEV), inp.q_seq.to(DEV), inp.q_pos.to(DEV), st.scores[:300], w_shared=True)
    torch.cuda.synchronize()
    g = st.scores[:300].cpu().numpy()
    ref = oracle.indexer_scores(u8(inp.iq), inp.iq_scale.numpy(), w0.numpy(), u8(inp.ik), inp.ik_scale.numpy(),
                                inp.q_pos.numpy(), ld=320, w_shared=True)
    mask = np.arange(320)[None, :] <= inp.q_pos.numpy()[:, None]
    A = indexer_abs_scale(inp.iq, inp.iq_scale, w0.expand(300, -1), inp.ik, inp.ik_scale, np.arange(300))
    A = np.concatenate([A, np.zeros((300, 20))], axis=1)
    assert (np.abs(g - ref)[mask] <= BOUND_C * A[mask] + 1e-30).all()
    assert (g[~mask] == 12345.0).all()


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("case", ["normal", "ties", "zeros", "short_rows", "wide", "odd_ld", "mid", "mid_ties",
                                  "split_ties", "split_mixed", "split_long", "max_row"])
def test_topk_bitexact_from_identical_scores(case):
    say(f"[topk] {case}")
    rng = np.random.default_rng(sum(map(ord, case)))
    n_q, ld, k = 300, 5000, 2048
    if case == "wide":
        n_q, ld, k = 40, 131072, 2048
    if case == "odd_ld":            # rows not 16-byte aligned: scalar loads
        n_q, ld, k = 50, 20001, 2048
    if case == "mid":               # register-resident rows of the 16K..32K variant
        n_q, ld, k = 64, 32768, 1000
    if case == "mid_ties":          # 32K rows whose threshold bin overflows the candidate list
        n_q, ld, k = 300, 32768, 2048
    if case in ("split_ties", "split_mixed"):   # few long rows: split over workgroups
        n_q, ld, k = 64, 40000, 333 if case == "split_ties" else 2048
    if case == "split_long":        # 128 rows whose two parts would exceed 32K: four parts instead
        n_q, ld, k = 128, 70000, 2048
    if case == "max_row":           # the longest row the ABI accepts (DSA_MAX_TOPK_ROW)
        n_q, ld, k = 8, 262144, 2048
    s = rng.standard_normal((n_q, ld)).astype(np.float32)
    if case in ("ties", "split_ties"):
        s = np.round(s * 2) / 2
    if case == "mid_ties":          # 23% of a row ties at the top value: more than the list holds
        s = np.round(np.minimum(s, 1.0) * 2) / 2
    if case == "zeros":
        s[:, ::2] = 0.0
        s[:, 1::4] = -0.0
    pos = rng.integers(0, ld, size=n_q).astype(np.int32)
    pos[:4] = [0, k - 1, k, ld - 1]
    if case == "short_rows":
        pos = rng.integers(0, 2 * k, size=n_q).astype(np.int32)
    if case == "split_mixed":       # one part, a few parts, and lengths at the part-count steps
        pos[4:20] = [2 * k - 1, 2 * k, 4 * k - 1, 4 * k, 4 * k + 1, 6 * k + 3, 8 * k - 2, 8 * k, 16 * k - 1, 16 * k,
                     16 * k + 5, 17 * k, 3 * k + 7, 5 * k - 3, 12345, 39999 - 1]
    if case == "ties":
        k = 333
    sd = torch.from_numpy(s).to(DEV)
    pd = torch.from_numpy(pos).to(DEV)
    idx = torch.full((n_q, k), -7, dtype=torch.int32, device=DEV)
    dsa.topk(sd, pd, k, idx)
    torch.cuda.synchronize()
    ref = oracle.topk(s, pos, k, n_threads=oracle_threads())
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    if dsa.topk_workspace_size(n_q, ld, k) > 0:
        # the same call without a workspace selects every row in one workgroup
        idx1 = torch.full((n_q, k), -7, dtype=torch.int32, device=DEV)
        assert dsa.lib().dsa_topk(sd.data_ptr(), ld, pd.data_ptr(), n_q, k, idx1.data_ptr(), None, 0, None) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx1.cpu().numpy(), ref)


@pytest.mark.parametrize("ld", [32, 64, 100, 128])
def test_topk_k_one_split_short_rows(ld):
    """k = 1 with a workspace: rows of 4..31 candidates are cut into parts that
    each still hold more than k scores, so every part leaves its survivor in the
    workspace and the merge sees no stale entries."""
    say(f"[topk] k=1 split, ld={ld}")
    rng = np.random.default_rng(ld)
    n_q, k = 40, 1
    s = rng.standard_normal((n_q, ld)).astype(np.float32)
    s[::3] = np.round(s[::3])                                   # ties
    pos = rng.integers(3, 31, n_q).astype(np.int32)
    pos[:4] = [3, 7, 8, 30]
    assert dsa.topk_workspace_size(n_q, ld, k) > 0
    ws = torch.full((dsa.topk_workspace_size(n_q, ld, k),), 0x5A, dtype=torch.uint8, device=DEV)  # stale bytes
    idx = torch.full((n_q, k), -7, dtype=torch.int32, device=DEV)
    dsa.topk(torch.from_numpy(s).to(DEV), torch.from_numpy(pos).to(DEV), k, idx, ws=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(s, pos, k))


def test_topk_k_one_and_all_equal():
    say("[topk] k=1 / all equal")
    s = np.zeros((3, 100), np.float32)
    s[1, 37] = 1.0
    s[2] = -np.arange(100, dtype=np.float32)
    pos = np.int32([99, 99, 50])
    for k in (1, 7):
        idx = torch.empty((3, k), dtype=torch.int32, device=DEV)
        dsa.topk(torch.from_numpy(s).to(DEV), torch.from_numpy(pos).to(DEV), k, idx)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(s, pos, k))


# ------------------------------------------------------------------ sparse MLA
def _mla_ref(inp, idx, rows, kv_fp8=False, st=None):
    q = inp.q if inp.q is not None else inp.q_chunk(0, inp.iq.shape[0])
    if kv_fp8:
        codes, scales = oracle.kv_quantize(bits16(inp.kv))
        return oracle.sparse_mla(bits16(q[rows]), codes, idx[rows], SM_SCALE, kv_scale=scales,
                                 n_threads=oracle_threads())
    return oracle.sparse_mla(bits16(q[rows]), bits16(inp.kv), idx[rows], SM_SCALE, n_threads=oracle_threads())


@pytest.mark.parametrize("base,L,paged,kv_fp8", [("C1", 1024, False, False), ("C1", 1024, True, True),
                                                 ("C2", 2304, True, False), ("C2", 2304, False, True),
                                                 ("C2", 333, False, False)])
def test_sparse_mla_prefill_vs_oracle(base, L, paged, kv_fp8):
    say(f"[mla prefill] {base} L={L} paged={paged} fp8={kv_fp8}")
    c = _cfg(base, paged=paged)
    inp = synth.make_prefill(c, L=L)
    st = run_prefill(inp, c.k, kv_fp8=kv_fp8)
    idx = st.idx.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, L, max(1, L // 40)), [L - 1], np.arange(min(L, c.k) - 2, min(L, c.k) + 2)]))
    rows = rows[(rows >= 0) & (rows < L)]
    ref_o, ref_l = _mla_ref(inp, idx, rows, kv_fp8)
    g_o = st.out[rows].float().cpu().numpy()
    g_l = st.lse[rows].cpu().numpy()
    e = max_abs_rel(g_o, ref_o)
    el = float(np.abs(g_l - ref_l).max())
    say(f"  out max-abs-rel = {e:.3e}, lse max abs err = {el:.3e}")
    assert e <= (TOL_FP8 if kv_fp8 else TOL_BF16)
    assert el <= 2e-2


@pytest.mark.parametrize("h,kv_fp8", [(16, False), (24, False), (40, True), (48, True), (64, False), (96, False),
                                       (112, True), (120, False)])
def test_sparse_mla_head_counts(h, kv_fp8):
    """Head counts other than 8 and 128 (1 to 4 waves, a partly used last wave;
    the supported set is the multiples of 8 up to 128):
    prefill and decode against the oracle on the same indices."""
    say(f"[mla heads] h={h} fp8={kv_fp8}")
    c = _cfg("C1", h=h, k=256)
    L = 700
    inp = synth.make_prefill(c, L=L)
    st = run_prefill(inp, c.k, kv_fp8=kv_fp8)
    idx = st.idx.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, L, 37), [L - 1, 255, 256]]))
    ref_o, ref_l = _mla_ref(inp, idx, rows, kv_fp8)
    tol = TOL_FP8 if kv_fp8 else TOL_BF16
    assert max_abs_rel(st.out[rows].float().cpu().numpy(), ref_o) <= tol
    assert float(np.abs(st.lse[rows].cpu().numpy() - ref_l).max()) <= 2e-2
    # the same rows through both decode forms: 3 splits, and one workgroup per
    # (query, 32 heads) with a partly used last head group
    d = lambda x: x.to(DEV)
    n = len(rows)
    for n_splits in (3, 1):
        need = dsa.sparse_mla_decode_workspace_size(n, h, c.k, n_splits)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        out2 = torch.empty((n, h, 512), dtype=torch.bfloat16, device=DEV)
        lse2 = torch.empty((n, h), dtype=torch.float32, device=DEV)
        dsa.sparse_mla_decode(d(inp.q[rows]), st.kv_cache, d(inp.kv_slot_table), torch.zeros(n, dtype=torch.int32,
                              device=DEV), st.idx[torch.from_numpy(rows).to(DEV)].contiguous(), SM_SCALE, out2, lse2,
                              kv_scale=st.kv_scale, n_splits=n_splits, ws=ws)
        torch.cuda.synchronize()
        assert max_abs_rel(out2.float().cpu().numpy(), ref_o) <= tol, n_splits
        assert float(np.abs(lse2.cpu().numpy() - ref_l).max()) <= 2e-2, n_splits


def _restart_inputs(case, n=4, h=128, k=512, seed=0):
    """Queries and latent rows whose logits jump far above each head's first 32
    selected rows, so the kernels' fixed softmax reference (the maximum over a
    head's first 32 rows, with 64 log2 units of headroom) has to be raised.
    q[t, h] = u_t + 0.7 noise; ordinary rows are N(0, 1), so their logits stay
    within a few log2 units of 0; a "hot" row beta u_t + 0.3 noise scores about
    34.6 beta log2 units (576 beta / 24 log2(e)).  Hot rows are placed at chosen
    positions of each query's selection (tiles of 64 rows in selection order):
      one: beta 2.5 / 2.45 at positions 100, 101 (tile 1) and 2.48 at 330: one
           raise, then a softmax shared by three rows;
      two: beta 2.5 at 100, then beta 5.0 at 450 (tile 7): raised twice.
    Queries select disjoint random rows; -1 entries pad nothing (k full)."""
    g = torch.Generator().manual_seed(7700 + seed + (0 if case == "one" else 50))
    N = n * k
    u = torch.randn((n, 576), generator=g)
    q = (u[:, None, :] + 0.7 * torch.randn((n, h, 576), generator=g)).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g)
    perm = torch.randperm(N, generator=g).reshape(n, k)
    idx = perm.clone()
    hot = {"one": [(100, 2.5), (101, 2.45), (330, 2.48)], "two": [(100, 2.5), (450, 5.0)]}[case]
    for t in range(n):
        for p, beta in hot:
            kv[int(idx[t, p])] = beta * u[t] + 0.3 * torch.randn(576, generator=g)
    kv = kv.to(torch.bfloat16)
    return q, kv, idx.to(torch.int32)


def _restart_raises(q, kv, idx, first=0, count=None):
    """Number of times the reference must move for the selection idx[first:first+count]
    (the kernels' rule, in float64 on the inputs): the first tile whose largest
    log2 logit exceeds the reference + 64 raises the reference to the largest
    logit seen up to that tile, and the scan starts over."""
    c2 = SM_SCALE / np.log(2.0)
    qd = q.double()
    kd = kv.double()
    n = q.shape[0]
    raises = []
    for t in range(n):
        sel = idx[t, first:first + (count or idx.shape[1])].long()
        lg = c2 * (qd[t] @ kd[sel].T)                       # [h, rows] log2 logits
        ref = lg[:, :32].max(dim=1).values
        r = 0
        while True:
            seen, moved = ref.clone(), False
            for j0 in range(0, lg.shape[1], 64):
                tm = lg[:, j0:j0 + 64].max(dim=1).values
                seen = torch.maximum(seen, tm)
                if (tm > ref + 64).any():
                    ref, moved = seen, True
                    break
            if not moved:
                break
            r += 1
        raises.append(r)
    return raises


@pytest.mark.parametrize("case", ["one", "two"])
@pytest.mark.parametrize("kv_fp8", [False, True])
def test_sparse_mla_softmax_reference_raised(case, kv_fp8):
    """The restart path of the sparse MLA kernels: logits far above the first
    rows' maximum make the kernels raise their softmax reference (once or twice)
    and start the query over; out and lse must still match the oracle.  Prefill
    form, and the split decode form with 1..4 splits (splits of 128 rows put the
    hot rows past each split's first 32 rows too)."""
    say(f"[mla] softmax reference raised: {case}, fp8={kv_fp8}")
    q, kv, idx = _restart_inputs(case)
    n, h, k = q.shape[0], q.shape[1], idx.shape[1]
    raises = _restart_raises(q, kv, idx)
    assert min(raises) >= (1 if case == "one" else 2), raises
    for s in (2, 4):       # the decode splits that hold hot rows past their first 32 rows raise too
        per = k // s
        assert max(sum(_restart_raises(q, kv, idx, p * per, per)) for p in range(s)) >= 1
    N = kv.shape[0]
    table = torch.arange(N, dtype=torch.int32, device=DEV).reshape(1, N)
    q_seq = torch.zeros(n, dtype=torch.int32, device=DEV)
    if kv_fp8:
        cache = torch.zeros((N, 576), dtype=torch.uint8, device=DEV)
        scale = torch.zeros(N, dtype=torch.float32, device=DEV)
        dsa.kv_cache_store(kv.to(DEV), torch.arange(N, dtype=torch.int64, device=DEV), cache, scale)
        codes, scales = oracle.kv_quantize(bits16(kv))
        ref_o, ref_l = oracle.sparse_mla(bits16(q), codes, idx.numpy(), SM_SCALE, kv_scale=scales)
    else:
        cache, scale = kv.to(DEV), None
        ref_o, ref_l = oracle.sparse_mla(bits16(q), bits16(kv), idx.numpy(), SM_SCALE)
    assert np.isfinite(ref_o).all()
    tol = TOL_FP8 if kv_fp8 else TOL_BF16
    out = torch.empty((n, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n, h), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_prefill(q.to(DEV), cache, table, q_seq, idx.to(DEV), SM_SCALE, out, lse, kv_scale=scale)
    torch.cuda.synchronize()
    e, el = max_abs_rel(out.float().cpu().numpy(), ref_o), float(np.abs(lse.cpu().numpy() - ref_l).max())
    say(f"  prefill: out max-abs-rel {e:.3e}, lse max abs err {el:.3e}; raises per query {raises}")
    assert e <= tol and el <= 2e-2
    for n_splits in (1, 2, 3, 4):
        need = dsa.sparse_mla_decode_workspace_size(n, h, k, n_splits)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        out.zero_()
        lse.zero_()
        dsa.sparse_mla_decode(q.to(DEV), cache, table, q_seq, idx.to(DEV), SM_SCALE, out, lse, kv_scale=scale,
                              n_splits=n_splits, ws=ws)
        torch.cuda.synchronize()
        e, el = max_abs_rel(out.float().cpu().numpy(), ref_o), float(np.abs(lse.cpu().numpy() - ref_l).max())
        say(f"  decode, {n_splits} splits: out max-abs-rel {e:.3e}, lse max abs err {el:.3e}")
        assert e <= tol and el <= 2e-2


def test_dense_degeneration_k_covers_all():
    """k >= L: every predecessor is selected and the output is dense causal MLA."""
    say("[dense degeneration] C1, k = L")
    c = CONFIGS["C1"]
    L = 512
    inp = synth.make_prefill(c, L=L)
    st = run_prefill(inp, L)
    idx = st.idx.cpu().numpy()
    exp = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], np.arange(L)[None, :], -1)
    np.testing.assert_array_equal(idx, exp)
    ref_o, ref_l = oracle.dense_mla(bits16(inp.q), bits16(inp.kv), inp.q_pos.numpy(), SM_SCALE,
                                    n_threads=oracle_threads())
    assert max_abs_rel(st.out.float().cpu().numpy(), ref_o) <= TOL_BF16


def test_single_index_gives_value_row():
    say("[mla] single index")
    c = CONFIGS["C2"]
    n, N = 16, 500
    q = synth.bf16_normal((n, c.h, 576), 911).to(DEV)
    kv = synth.bf16_normal((N, 576), 912)
    kv_cache = kv.to(DEV)
    table = torch.arange(N, dtype=torch.int32, device=DEV).reshape(1, N)
    idx = torch.full((n, 64), -1, dtype=torch.int32)
    sel = torch.randint(0, N, (n,), generator=synth.gen(913))
    idx[:, 0] = sel
    idx[3, :] = -1
    idx[3, 40] = int(sel[3])                             # a lone index in the middle of the list
    out = torch.empty((n, c.h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n, c.h), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_prefill(q, kv_cache, table, torch.zeros(n, dtype=torch.int32, device=DEV), idx.to(DEV),
                           SM_SCALE, out, lse)
    torch.cuda.synchronize()
    got = bits16(out).reshape(n, c.h, 512)
    for t in range(n):
        np.testing.assert_array_equal(got[t], np.broadcast_to(bits16(kv[sel[t]])[:512], (c.h, 512)))


def test_single_index_fp8_cache_every_code():
    """One selected row of an FP8 cache: the output is that row's 512 value codes
    times its scale, for every finite E4M3 code (powers-of-two scales keep the
    product exact in bf16), i.e. the in-kernel expansion of each code is exact."""
    say("[mla] single index, FP8 cache, all codes")
    c = CONFIGS["C2"]
    n, N = 4, 8
    codes = (np.arange(N * 576) * 37 % 256).astype(np.uint8).reshape(N, 576)   # every code in every row's values
    codes[codes == 0x7F] = 0x7E                                                 # no NaN codes
    codes[codes == 0xFF] = 0xFE
    assert all(len(np.unique(codes[r, :512])) == 254 for r in range(N))
    scales = np.array([2.0 ** e for e in (-4, 0, 3, -1, 1, 2, -2, 5)], dtype=np.float32)
    cache = torch.from_numpy(codes).to(DEV)
    kv_scale = torch.from_numpy(scales).to(DEV)
    q = synth.bf16_normal((n, c.h, 576), 915).to(DEV)
    table = torch.arange(N, dtype=torch.int32, device=DEV).reshape(1, N)
    sel = [5, 0, 2, 7]
    idx = torch.full((n, 64), -1, dtype=torch.int32)
    idx[:, 0] = torch.tensor(sel, dtype=torch.int32)
    out = torch.empty((n, c.h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n, c.h), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_prefill(q, cache, table, torch.zeros(n, dtype=torch.int32, device=DEV), idx.to(DEV),
                           SM_SCALE, out, lse, kv_scale=kv_scale)
    torch.cuda.synchronize()
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()              # exact decode of each code
    for t, r in enumerate(sel):
        want = (dec[r, :512] * float(scales[r]) + 0.0).to(torch.bfloat16)        # -0 accumulates to +0
        np.testing.assert_array_equal(bits16(out[t].cpu()), np.broadcast_to(bits16(want), (c.h, 512)))


def test_empty_selection_and_out_of_range_entries():
    say("[mla] empty / out-of-range entries")
    n, N, h = 4, 100, 16
    q = synth.bf16_normal((n, h, 576), 921).to(DEV)
    kv = synth.bf16_normal((N, 576), 922)
    table = torch.arange(N, dtype=torch.int32).reshape(1, N)
    table[0, 7] = 10 ** 6                                # slot outside the cache -> skipped
    idx = torch.full((n, 32), -1, dtype=torch.int32)
    idx[1, :3] = torch.tensor([5, 7, 500])               # 7 -> bad slot, 500 -> past the table
    idx[2, :2] = torch.tensor([5, 6])
    out = torch.empty((n, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n, h), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_prefill(q, kv.to(DEV), table.to(DEV), torch.zeros(n, dtype=torch.int32, device=DEV),
                           idx.to(DEV), SM_SCALE, out, lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert (o[0] == 0).all() and (o[3] == 0).all() and np.isneginf(lse.cpu().numpy()[[0, 3]]).all()
    np.testing.assert_array_equal(bits16(out)[1], np.broadcast_to(bits16(kv[5])[:512], (h, 512)))
    ref_o, _ = oracle.sparse_mla(bits16(q.cpu()[2:3]), bits16(kv), idx[2:3].numpy(), SM_SCALE)
    assert max_abs_rel(o[2:3], ref_o) <= TOL_BF16


# ------------------------------------------------------------------ invariants
def test_page_permutation_invariance():
    """Identity vs shuffled page / slot layouts give bit-identical results."""
    say("[invariance] page permutation")
    L = 2000
    a = run_prefill(synth.make_prefill(_cfg("C2", paged=False), L=L), 2048)
    b = run_prefill(synth.make_prefill(_cfg("C2", paged=True), L=L), 2048)
    causal = torch.arange(L, device=DEV)[None, :] <= torch.arange(L, device=DEV)[:, None]
    assert torch.equal(a.scores[causal], b.scores[causal])      # columns past q_pos are never written
    assert torch.equal(a.idx, b.idx)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))


def test_chunked_equals_monolithic():
    """Chunked prefill against the growing cache reproduces the monolithic rows."""
    say("[invariance] chunked == monolithic (fp8 kv)")
    c = _cfg("C5", L=3072, chunk=1024)
    inp = synth.make_prefill(c, L=3072, materialize_q=False)
    mono = run_prefill(inp, c.k, kv_fp8=True)
    st = P.alloc_prefill(inp.n_pages, c.d_i, inp.n_slots, c.chunk, 3072, c.k, c.h, kv_fp8=True)
    d = lambda x: x.to(DEV)
    for c0 in range(0, 3072, c.chunk):
        c1 = c0 + c.chunk
        P.store_tokens(st, d(inp.ik[c0:c1]), d(inp.ik_scale[c0:c1]), d(inp.ik_slot[c0:c1]), d(inp.kv[c0:c1]),
                       d(inp.kv_slot_table[0, c0:c1]).long())
        P.prefill_step(st, d(inp.iq[c0:c1]), d(inp.iq_scale[c0:c1]), d(inp.w[c0:c1]), d(inp.page_table),
                       d(inp.kv_slot_table), d(inp.q_seq[c0:c1]), d(inp.q_pos[c0:c1]), d(inp.q_chunk(c0, c1)),
                       c.k, SM_SCALE)
        torch.cuda.synchronize()
        m = inp.q_pos[c0:c1].numpy()
        sc_chunk = st.scores.cpu().numpy()
        sc_mono = mono.scores[c0:c1].cpu().numpy()
        mask = np.arange(3072)[None, :] <= m[:, None]
        assert np.array_equal(sc_chunk[mask], sc_mono[mask])
        assert torch.equal(st.idx, mono.idx[c0:c1])
        assert torch.equal(st.out.view(torch.int16), mono.out[c0:c1].view(torch.int16))


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("batch,lo,hi,n_splits,kv_fp8,m", [(8, 2000, 9000, 0, False, 1), (5, 100, 3000, 3, False, 1),
                                                           (3, 2049, 2049, 1, False, 1), (6, 1500, 7000, 0, True, 1),
                                                           (4, 2049, 4100, 2, True, 1), (5, 1900, 6000, 0, False, 3),
                                                           (4, 2050, 2052, 2, True, 2), (8, 100, 3000, 1, False, 1),
                                                           (6, 1500, 7000, 1, True, 1), (5, 1900, 6000, 1, False, 3),
                                                           (7, 2041, 2100, 1, True, 2)])
def test_decode_vs_oracle(batch, lo, hi, n_splits, kv_fp8, m):
    """m query tokens per sequence (m > 1: the multi-token-prediction shape).
    n_splits = 1: one workgroup per (query, 32 heads) over the whole selection
    (contexts below k leave waves with few or no rows); 2, 3: split index lists
    merged by a second launch; 0: the automatic choice."""
    say(f"[decode] B={batch} ctx=[{lo},{hi}] splits={n_splits} fp8={kv_fp8} queries/seq={m}")
    c = CONFIGS["C4"]
    inp = synth.make_decode(c, batch=batch, ctx_lo=lo, ctx_hi=hi, queries_per_seq=m)
    d = lambda x: x.to(DEV)
    caches = P.alloc_prefill(inp.n_pages, c.d_i, inp.n_slots, 1, 1, c.k, c.h, kv_fp8=kv_fp8)
    kv_slot = torch.empty(inp.n_slots, dtype=torch.int64)
    for b in range(batch):
        s0, nb = int(inp.seq_start[b]), int(inp.lens[b])
        kv_slot[s0:s0 + nb] = inp.kv_slot_table[b, :nb].long()
    P.store_tokens(caches, d(inp.ik), d(inp.ik_scale), d(inp.ik_slot), d(inp.kv), d(kv_slot))
    ld = int(inp.lens.max())
    ds = P.alloc_decode(batch * m, ld, c.k, c.h, n_splits=n_splits)
    P.decode_step(ds, caches, d(inp.iq), d(inp.iq_scale), d(inp.w), d(inp.page_table), d(inp.kv_slot_table),
                  d(inp.q_seq), d(inp.q_pos), d(inp.q), c.k, SM_SCALE)
    torch.cuda.synchronize()
    g = ds.scores.cpu().numpy()
    pos = inp.q_pos.numpy()
    ref = oracle.indexer_scores(u8(inp.iq), inp.iq_scale.numpy(), inp.w.numpy(), u8(inp.ik), inp.ik_scale.numpy(),
                                pos, seq_start=inp.seq_start.numpy(), q_seq=inp.q_seq.numpy(), ld=ld,
                                n_threads=oracle_threads())
    mask = np.arange(ld)[None, :] <= pos[:, None]
    for t in range(batch * m):
        b = int(inp.q_seq[t])
        s0, nk = int(inp.seq_start[b]), int(pos[t]) + 1
        A = indexer_abs_scale(inp.iq[t:t + 1], inp.iq_scale[t:t + 1], inp.w[t:t + 1], inp.ik[s0:s0 + nk],
                              inp.ik_scale[s0:s0 + nk], np.arange(1))
        assert (np.abs(g[t, :nk] - ref[t, :nk]) <= BOUND_C * A[0] + 1e-30).all(), t
    np.testing.assert_array_equal(ds.idx.cpu().numpy(), oracle.topk(g, pos, c.k))
    idx = ds.idx.cpu().numpy()
    if kv_fp8:
        codes, scales = oracle.kv_quantize(bits16(inp.kv))
        ref_o, ref_l = oracle.sparse_mla(bits16(inp.q), codes, idx, SM_SCALE, kv_scale=scales,
                                         seq_start=inp.seq_start.numpy(), q_seq=inp.q_seq.numpy(),
                                         n_threads=oracle_threads())
    else:
        ref_o, ref_l = oracle.sparse_mla(bits16(inp.q), bits16(inp.kv), idx, SM_SCALE,
                                         seq_start=inp.seq_start.numpy(), q_seq=inp.q_seq.numpy(),
                                         n_threads=oracle_threads())
    tol = TOL_FP8 if kv_fp8 else TOL_BF16
    e = max_abs_rel(ds.out.float().cpu().numpy(), ref_o)
    say(f"  decode out max-abs-rel = {e:.3e}")
    assert e <= tol
    assert float(np.abs(ds.lse.cpu().numpy() - ref_l).max()) <= 2e-2
    # the prefill-form kernel on the same indices agrees within tolerance
    out2 = torch.empty_like(ds.out)
    dsa.sparse_mla_prefill(d(inp.q), caches.kv_cache, d(inp.kv_slot_table), d(inp.q_seq), ds.idx, SM_SCALE, out2,
                           kv_scale=caches.kv_scale)
    torch.cuda.synchronize()
    assert max_abs_rel(out2.float().cpu().numpy(), ref_o) <= tol


def test_decode_row_matches_prefill_row():
    """A decode query at position N-1 equals the last prefill row of the same sequence."""
    say("[invariance] decode row == prefill row")
    c = _cfg("C2", paged=True)
    L = 3000
    inp = synth.make_prefill(c, L=L)
    st = run_prefill(inp, c.k)
    d = lambda x: x.to(DEV)
    ds = P.alloc_decode(1, L, c.k, c.h)
    P.decode_step(ds, st, d(inp.iq[-1:]), d(inp.iq_scale[-1:]), d(inp.w[-1:]), d(inp.page_table),
                  d(inp.kv_slot_table), d(inp.q_seq[-1:]), d(inp.q_pos[-1:]), d(inp.q[-1:]), c.k, SM_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(ds.scores[0, :L], st.scores[L - 1])      # same per-pair arithmetic in both indexers
    assert torch.equal(ds.idx[0], st.idx[L - 1])
    assert max_abs_rel(ds.out[0].float().cpu().numpy(), st.out[L - 1].float().cpu().numpy()) <= 1e-2


def test_decode_graph_replay_matches_eager():
    """The decode step captured as a HIP graph replays to the eager result, bit for bit,
    on every replay (eager work and synchronizations between the replays)."""
    say("[graph] decode step captured and replayed")
    c = CONFIGS["C4"]
    inp = synth.make_decode(c, batch=6, ctx_lo=2100, ctx_hi=7000, queries_per_seq=2)
    d = lambda x: x.to(DEV)
    caches = P.alloc_prefill(inp.n_pages, c.d_i, inp.n_slots, 1, 1, c.k, c.h)
    kv_slot = torch.empty(inp.n_slots, dtype=torch.int64)
    for b in range(6):
        s0, nb = int(inp.seq_start[b]), int(inp.lens[b])
        kv_slot[s0:s0 + nb] = inp.kv_slot_table[b, :nb].long()
    P.store_tokens(caches, d(inp.ik), d(inp.ik_scale), d(inp.ik_slot), d(inp.kv), d(kv_slot))
    args = [d(inp.iq), d(inp.iq_scale), d(inp.w), d(inp.page_table), d(inp.kv_slot_table), d(inp.q_seq),
            d(inp.q_pos), d(inp.q)]
    ld = int(inp.lens.max())
    ds = P.alloc_decode(12, ld, c.k, c.h)
    step = lambda st: P.decode_step(st, caches, *args, c.k, SM_SCALE)
    step(ds)
    torch.cuda.synchronize()
    ref = [ds.idx.clone(), ds.out.clone(), ds.lse.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(ds)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(ds)
    other = P.alloc_decode(12, ld, c.k, c.h)
    for r in range(3):
        ds.idx.fill_(-7)
        ds.out.zero_()
        ds.lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        step(other)                      # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(ref, (ds.idx, ds.out, ds.lse)):
            assert torch.equal(a, b), r
        for a, b in zip(ref, (other.idx, other.out, other.lse)):
            assert torch.equal(a, b), r


# ------------------------------------------------------------------ fused indexer -> top-k (decode form)
def _decode_keys(batch, lo, hi, m):
    """Seeded decode inputs (queries at the last m positions) and the indexer key cache."""
    c = CONFIGS["C4"]
    inp = synth.make_decode(c, batch=batch, ctx_lo=lo, ctx_hi=hi, queries_per_seq=m, device=DEV)
    key_cache = torch.zeros((inp.n_pages, 64, c.d_i), dtype=torch.uint8, device=DEV)
    key_scale = torch.zeros((inp.n_pages, 64), dtype=torch.float32, device=DEV)
    dsa.indexer_cache_store(inp.ik, inp.ik_scale, inp.ik_slot, key_cache, key_scale)
    return inp, key_cache, key_scale


def _two_calls(inp, key_cache, key_scale, table, ld, k):
    n_q = inp.iq.shape[0]
    sc = torch.full((n_q, ld), -7.0, device=DEV)
    idx = torch.full((n_q, k), -9, dtype=torch.int32, device=DEV)
    dsa.indexer_scores(inp.iq, inp.iq_scale, inp.w, key_cache, key_scale, table, inp.q_seq, inp.q_pos, sc)
    need = dsa.topk_workspace_size(n_q, ld, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    dsa.topk(sc, inp.q_pos, k, idx, ws=ws if need else None)
    return sc, idx


FUSED_ROW_BYTES, FUSED_ZERO_BYTES = 106560, 8256


def _fused_zero_regions_clear(ws):
    """Every row block's leading region (histogram and counters) is zero again."""
    rows = ws.numel() // FUSED_ROW_BYTES
    return int(ws[: rows * FUSED_ROW_BYTES].view(rows, FUSED_ROW_BYTES)[:, :FUSED_ZERO_BYTES].count_nonzero()) == 0


def _fused(inp, key_cache, key_scale, table, ld, k, ws):
    n_q = inp.iq.shape[0]
    sc = torch.full((n_q, ld), -7.0, device=DEV)
    idx = torch.full((n_q, k), -9, dtype=torch.int32, device=DEV)
    dsa.indexer_topk(inp.iq, inp.iq_scale, inp.w, key_cache, key_scale, table, inp.q_seq, inp.q_pos, sc, k, idx, ws)
    return sc, idx


@pytest.mark.parametrize("batch,lo,hi,m,k,variant", [
    (8, 2000, 9000, 1, 2048, "plain"),          # rows held in registers
    (4, 33000, 70000, 1, 2048, "plain"),        # rows longer than 32K: streamed
    (6, 1500, 20000, 2, 2048, "plain"),         # query pairs of one sequence share the scan
    (8, 100, 3000, 1, 2048, "plain"),           # contexts below k: every candidate kept
    (5, 5000, 9000, 1, 1, "plain"),
    (5, 5000, 9001, 1, 64, "odd_ld"),           # rows not 16-byte aligned
    (4, 9000, 40000, 1, 2048, "short_table"),   # pages past the table: NaN scores
    (3, 9000, 12000, 1, 2048, "ties"),          # all scores equal: the threshold bin overflows the list
    (2, 40000, 50000, 1, 512, "ties"),          # ... in streamed rows
    (2, 120000, 131072, 1, 2048, "plain"),      # the longest decode contexts: 8 parts per row
    (2, 65536, 65536, 1, 2048, "plain"),        # rows of exactly 4 parts
    (2, 262144, 262144, 1, 2048, "plain"),      # the longest row accepted (16 parts)
    (128, 1500, 9000, 2, 2048, "plain"),        # 256 queries: the most the fused call takes
])
def test_indexer_topk_fused_matches_two_calls(batch, lo, hi, m, k, variant):
    """dsa_indexer_topk writes the same scores and indices, bit for bit, as
    dsa_indexer_scores followed by dsa_topk; the indices equal the oracle's top-k
    of those scores; the workspace's histogram and counters are zero again after
    every call, so a second call (fewer queries, same workspace) is exact too."""
    say(f"[fused] B={batch} ctx=[{lo},{hi}] queries/seq={m} k={k} {variant}")
    inp, key_cache, key_scale = _decode_keys(batch, lo, hi, m)
    if variant == "ties":
        inp = dataclasses.replace(inp, w=torch.zeros_like(inp.w))
    ld = int(inp.lens.max())
    if variant == "odd_ld":
        ld |= 1
    table = inp.page_table
    if variant == "short_table":
        table = table[:, :100].contiguous()
    n_q = inp.iq.shape[0]
    ws = torch.zeros(dsa.indexer_topk_workspace_size(n_q), dtype=torch.uint8, device=DEV)
    sa, ia = _two_calls(inp, key_cache, key_scale, table, ld, k)
    sb, ib = _fused(inp, key_cache, key_scale, table, ld, k, ws)
    torch.cuda.synchronize()
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    assert torch.equal(ia, ib)
    assert _fused_zero_regions_clear(ws)
    g = sb.cpu().numpy()
    pos = inp.q_pos.cpu().numpy()
    if variant == "short_table":
        assert np.isnan(g[0, 6400:pos[0] + 1]).all()
    else:
        np.testing.assert_array_equal(ib.cpu().numpy(), oracle.topk(g, pos, k))
    # a second call on the same (zero again) workspace, fewer queries
    half = dataclasses.replace(inp, iq=inp.iq[: n_q // 2 + 1], iq_scale=inp.iq_scale[: n_q // 2 + 1],
                               w=inp.w[: n_q // 2 + 1], q_seq=inp.q_seq[: n_q // 2 + 1],
                               q_pos=inp.q_pos[: n_q // 2 + 1])
    sc2, ic2 = _fused(half, key_cache, key_scale, table, ld, k, ws)
    torch.cuda.synchronize()
    assert torch.equal(ic2, ia[: n_q // 2 + 1])
    assert torch.equal(sc2.view(torch.int32), sa[: n_q // 2 + 1].view(torch.int32))
    assert _fused_zero_regions_clear(ws)


def test_indexer_topk_fused_graph_replay():
    """The fused call captured in a HIP graph: every replay (eager fused calls on
    the same workspace in between) gives the eager indices, and the workspace's
    histogram and counters are zero after each."""
    say("[fused] graph replay")
    inp, key_cache, key_scale = _decode_keys(6, 3000, 40000, 1)
    ld, k, n_q = int(inp.lens.max()), 2048, 6
    ws = torch.zeros(dsa.indexer_topk_workspace_size(n_q), dtype=torch.uint8, device=DEV)
    sc = torch.zeros((n_q, ld), device=DEV)
    idx = torch.zeros((n_q, k), dtype=torch.int32, device=DEV)
    call = lambda: dsa.indexer_topk(inp.iq, inp.iq_scale, inp.w, key_cache, key_scale, inp.page_table, inp.q_seq,
                                    inp.q_pos, sc, k, idx, ws)
    call()
    torch.cuda.synchronize()
    ref = idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), r
        assert _fused_zero_regions_clear(ws), r
        call()                          # eager work on the same workspace between the replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), r


def _crafted_rows(values):
    """Indexer inputs whose scores are exactly `values` [n_q, n]: one weighted head,
    q = e_0 (FP8 1.0), key s = values[., s] in dimension 0 (FP8), unit scales;
    query r is the last token of sequence r (identity page tables)."""
    n_q, n = values.shape
    pages = (n + 63) // 64
    codes = torch.from_numpy(values.astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(codes.float().numpy(), values.astype(np.float32)), "not exactly representable"
    ik = torch.zeros((n_q * pages * 64, 128), dtype=torch.uint8)
    for r in range(n_q):
        ik[r * pages * 64: r * pages * 64 + n, 0] = codes[r].view(torch.uint8)
    key_cache = torch.zeros((n_q * pages, 64, 128), dtype=torch.uint8, device=DEV)
    key_scale = torch.zeros((n_q * pages, 64), dtype=torch.float32, device=DEV)
    dsa.indexer_cache_store(ik.to(DEV), torch.ones(ik.shape[0], device=DEV),
                            torch.arange(ik.shape[0], dtype=torch.int64, device=DEV), key_cache, key_scale)
    iq = torch.zeros((n_q, 64, 128), dtype=torch.uint8)
    iq[:, 0, 0] = 0x38                                          # E4M3 1.0
    w = torch.zeros((n_q, 64))
    w[:, 0] = 1.0
    table = torch.arange(n_q * pages, dtype=torch.int32).reshape(n_q, pages)
    inp = dataclasses.make_dataclass("Crafted", ["iq", "iq_scale", "w", "q_seq", "q_pos", "page_table"])(
        iq.to(DEV), torch.ones(n_q, device=DEV), w.to(DEV), torch.arange(n_q, dtype=torch.int32, device=DEV),
        torch.full((n_q,), n - 1, dtype=torch.int32, device=DEV), table.to(DEV))
    return inp, key_cache, key_scale


@pytest.mark.parametrize("pattern", ["wave_overflow", "spread_ties", "big_bin", "whole_bin", "last_part_one_key"])
def test_indexer_topk_fused_crafted_scores(pattern):
    """Score rows built to reach each path of the fused selection (parts of 32768
    scores, 16 waves of a part each owning 256 of every 4096): the threshold bin's
    keys crowded into one wave's slots (its list overflows), spread ties (the
    list path), a bin larger than the list (the whole row re-read), a bin taken
    whole, and a last part of one score.  Indices equal the two calls' and the
    oracle's, bit for bit."""
    say(f"[fused] crafted scores: {pattern}")
    rng = np.random.default_rng(sum(map(ord, pattern)))
    n, k = (40000, 1000) if pattern != "last_part_one_key" else (65537, 2048)
    vals = np.full((2, n), 0.5)
    for r in range(2):
        if pattern == "wave_overflow":          # wave 0's slots of every chunk of part 0
            pos = (np.arange(8)[:, None] * 4096 + np.arange(256)[None, :]).ravel()
            vals[r, pos] = rng.choice([2.0, 2.25], size=pos.size)
        elif pattern == "spread_ties":
            pos = rng.choice(n, 5000, replace=False)
            vals[r, pos] = rng.choice([2.0, 2.25], size=pos.size)
        elif pattern == "big_bin":
            pos = rng.choice(n, 10000, replace=False)
            vals[r, pos] = rng.choice([2.0, 2.25], size=pos.size)
        elif pattern == "whole_bin":
            perm = rng.permutation(n)
            vals[r, perm[:k]] = 4.0
            vals[r, perm[k:k + 3000]] = np.where(rng.random(3000) < 0.5, 0.75, 1.0)
        else:                                   # the row's last score is the only one of part 2
            codes = torch.from_numpy(rng.integers(0x20, 0x70, size=n).astype(np.uint8))
            vals[r] = codes.view(torch.float8_e4m3fn).double().numpy()
            vals[r, -1] = 448.0
    inp, key_cache, key_scale = _crafted_rows(vals)
    ws = torch.zeros(dsa.indexer_topk_workspace_size(2), dtype=torch.uint8, device=DEV)
    sa, ia = _two_calls(inp, key_cache, key_scale, inp.page_table, n, k)
    sb, ib = _fused(inp, key_cache, key_scale, inp.page_table, n, k, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sb.cpu().numpy(), vals.astype(np.float32))
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    want = oracle.topk(vals.astype(np.float32), np.full(2, n - 1), k)
    np.testing.assert_array_equal(ib.cpu().numpy(), want)
    np.testing.assert_array_equal(ia.cpu().numpy(), want)
    assert _fused_zero_regions_clear(ws)
    if pattern == "last_part_one_key":
        assert (ib.cpu().numpy() == n - 1).any(axis=1).all()
