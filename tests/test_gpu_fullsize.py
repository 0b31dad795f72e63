"""GPU parity at the full workload sizes.

Each workload runs exactly as the benchmark launches it (same input
generation, same calls, same launch geometry):
  * 8K prefill  (B=1, L=8192, k=2048, 64x128 FP8 indexer, 128-head MLA),
    plus the same shape in the exact-arithmetic regime E1: every row is
    verified (indexer row, its top-k, its MLA output);
  * 32K prefill (L=32768, shuffled 64-token pages and KV slots): at least 512
    stratified rows verified completely;
  * decode      (64 sequences, contexts ~ U[32768, 131072], one query each):
    every sequence's indexer row, top-k and MLA output;
  * chunked prefill of one 131072-token sequence in 8192-token chunks with
    an FP8 (E4M3 + per-token scale) latent cache: at least 512 stratified
    rows (32 per chunk) verified completely.
The stratified samples take rows below k (where the selection keeps every
candidate), rows at the top-k boundary, 64-token page boundaries, chunk
boundaries, the last rows and uniform picks.

Index parity: top-k on the GPU's own scores is bit-exact against the oracle
(every row); every GPU score is within 2^-15 * sum|terms| of the exact
score (the FP8 MFMA's bound on N(0, 1) inputs, measured in
test_gpu_numerics.py); end-to-end indices against the oracle's own
scores may differ only at near-ties inside that bound.  MLA outputs are
compared with the oracle on the GPU's own indices.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from synth.configs import CONFIGS, SM_SCALE
from gpu_common import DEV, say, bits16, u8, oracle_threads, key_cache_rows

pytestmark = pytest.mark.gpu

BOUND_C = 2.0 ** -15     # the FP8 MFMA's measured bound on these inputs (test_gpu_numerics.py)
TOL_BF16, TOL_FP8 = 2e-2, 5e-2
MIN_ROWS = 512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import long_context_sparse_fp8_amd as dsa
    dsa.lib()
    yield
    torch.cuda.empty_cache()


def _stratified_rows(L, k, n_min, seed, extra=()):
    """At least n_min distinct rows of [0, L): rows below and around k, 64-token
    page boundaries, the last rows, `extra`, then uniform picks."""
    rng = np.random.default_rng(seed)
    r = {0, 1, 2, 3, k - 2, k - 1, k, k + 1, L - 3, L - 2, L - 1, *extra}
    r |= set(rng.integers(0, min(k, L), 48).tolist())                      # fewer candidates than k
    pages = rng.integers(1, L // 64, 32) * 64
    r |= set(pages.tolist()) | set((pages - 1).tolist())                   # page boundaries
    r |= set(range(L - 16, L))
    r = {x for x in r if 0 <= x < L}
    while len(r) < n_min:
        r |= set(rng.integers(0, L, n_min - len(r)).tolist())
    return np.array(sorted(r), dtype=np.int64)


def _abs_scale(iq, iqs, w, ik, iks):
    """A[r, s] = qs_r ks_s sum_j |w_rj| sum_i |q_rji k_si| (float64, host tensors)."""
    qv = np.abs(torch.from_numpy(u8(iq)).view(torch.float8_e4m3fn).double().numpy())   # [r, H, D]
    kv = np.abs(torch.from_numpy(u8(ik)).view(torch.float8_e4m3fn).double().numpy())   # [N, D]
    v = np.einsum("rh,rhd->rd", np.abs(w.double().numpy()), qv)
    return (v @ kv.T) * iqs.double().numpy()[:, None] * iks.double().numpy()[None, :]


class IndexStats:
    def __init__(self):
        self.rows = 0
        self.ratio = 0.0
        self.mism = 0

    def __str__(self):
        return (f"{self.rows} rows: indexer max |gpu-exact| / (2^-15 sum|terms|) {self.ratio:.4f}; "
                f"end-to-end index differences (near-ties) {self.mism}")


def _check_index_rows(stats, g_scores, ref_scores, A, pos, k, g_idx):
    """g_scores / ref_scores / A: [r, >= pos+1] for some rows; g_idx [r, k].
    1) top-k on the GPU's scores is bit-exact (oracle.topk on identical inputs);
    2) GPU scores are within BOUND_C * A of the exact scores;
    3) end-to-end indices differ from the oracle's only at near-ties."""
    ld = g_scores.shape[1]
    mask = np.arange(ld)[None, :] <= pos[:, None]
    np.testing.assert_array_equal(g_idx, oracle.topk(np.where(mask, g_scores, 0.0).astype(np.float32), pos, k,
                                                     n_threads=oracle_threads()))
    err = np.abs(g_scores.astype(np.float64) - ref_scores)[mask]
    ratio = float((err / (BOUND_C * A[mask] + 1e-300)).max())
    assert ratio <= 1.0, f"indexer error {ratio:.3f} x the bound"
    r_idx = oracle.topk(np.where(mask, ref_scores, 0.0).astype(np.float32), pos, k, n_threads=oracle_threads())
    for r in range(len(pos)):
        G = set(g_idx[r][g_idx[r] >= 0].tolist())
        R = set(r_idx[r][r_idx[r] >= 0].tolist())
        if G == R:
            continue
        gr, rg = np.array(sorted(G - R)), np.array(sorted(R - G))
        assert len(gr) == len(rg)
        stats.mism += len(gr)
        d = BOUND_C * A[r]
        # every swapped pair must be a near-tie: the GPU could rank s above r only if
        # their exact scores are within the two error bounds of each other
        lo_r = (ref_scores[r, rg] - d[rg]).min()
        hi_s = (ref_scores[r, gr] + d[gr]).max()
        assert (ref_scores[r, gr] + d[gr] >= lo_r).all() and (ref_scores[r, rg] - d[rg] <= hi_s).all(), \
            f"row {r}: index swap that is not a near-tie"
    stats.rows += len(pos)
    stats.ratio = max(stats.ratio, ratio)


class RelErr:
    """max |gpu - ref| / max |ref| accumulated over blocks of one output tensor."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.lse = 0.0

    def add(self, g, ref, g_lse, ref_lse):
        self.num = max(self.num, float(np.abs(np.asarray(g, np.float64) - ref).max()))
        self.den = max(self.den, float(np.abs(ref).max()))
        self.lse = max(self.lse, float(np.abs(np.asarray(g_lse, np.float64) - ref_lse).max()))

    @property
    def rel(self):
        return self.num / self.den if self.den > 0 else self.num


def _sel(t, rows):
    """Rows of a (device) tensor picked by a numpy index array, copied to the host."""
    return t[torch.as_tensor(np.asarray(rows), device=t.device)].cpu()


def _indexer_ref(iq, iqs, w, ik, iks, pos, ld=None):
    return oracle.indexer_scores(u8(iq), iqs.numpy(), w.numpy(), u8(ik), iks.numpy(), pos,
                                 ld=ld or int(pos.max()) + 1, n_threads=oracle_threads())


def _kv_ref(inp, kv_fp8):
    """The latent rows the oracle attends over: bf16 bits, or (for an FP8 cache)
    the oracle quantizer's codes and scales."""
    if kv_fp8:
        codes, scales = oracle.kv_quantize(bits16(inp.kv))
        return codes, scales
    return bits16(inp.kv), None


def _verify_prefill_rows(stats, rel, inp, kv_ref, rows, g_scores, g_idx, g_out, g_lse, q_rows, k, block=256):
    """Verify the given rows of one prefill sequence completely, in blocks: the
    indexer row, its top-k, and its MLA output (on the GPU's indices)."""
    ik, iks = inp.ik.cpu(), inp.ik_scale.cpu()
    kv, kv_scale = kv_ref
    for b0 in range(0, len(rows), block):
        r = rows[b0:b0 + block]
        pos = inp.q_pos.cpu().numpy()[r].astype(np.int32)
        ld = int(pos.max()) + 1
        iq, iqs, w = _sel(inp.iq, r), _sel(inp.iq_scale, r), _sel(inp.w, r)
        ref = _indexer_ref(iq, iqs, w, ik[:ld], iks[:ld], pos, ld)
        A = _abs_scale(iq, iqs, w, ik[:ld], iks[:ld])
        gi = g_idx[b0:b0 + block]
        _check_index_rows(stats, g_scores[b0:b0 + block, :ld], ref.astype(np.float64), A, pos, k, gi)
        ro, rl = oracle.sparse_mla(bits16(q_rows[b0:b0 + block]), kv, gi, SM_SCALE, kv_scale=kv_scale,
                                   n_threads=oracle_threads())
        rel.add(g_out[b0:b0 + block], ro, g_lse[b0:b0 + block], rl)


# ------------------------------------------------------------------ 8K prefill: every row
@pytest.mark.timeout(900)
@pytest.mark.parametrize("exact", [False, True])
def test_prefill_8k_full(exact):
    from long_context_sparse_fp8_amd import pipeline as P
    cfg = CONFIGS["C2"]
    say(f"[full C2] L={cfg.L} k={cfg.k} exact={exact}: every row")
    inp = synth.make_prefill(cfg, device=DEV, exact=exact)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, cfg.L, cfg.L, cfg.k, cfg.h)
    P.store_tokens(st, inp.ik, inp.ik_scale, inp.ik_slot, inp.kv, inp.kv_slot_table[0].long())
    P.prefill_step(st, inp.iq, inp.iq_scale, inp.w, inp.page_table, inp.kv_slot_table, inp.q_seq, inp.q_pos,
                   inp.q, cfg.k, SM_SCALE)
    torch.cuda.synchronize()
    L, k = cfg.L, cfg.k
    rows = np.arange(L)
    g_all = st.scores.cpu().numpy()
    gi_all = st.idx.cpu().numpy()
    if exact:
        # E1: scores and indices bit-exact on every row
        ik, iks = inp.ik.cpu(), inp.ik_scale.cpu()
        for b0 in range(0, L, 1024):
            r = rows[b0:b0 + 1024]
            pos = r.astype(np.int32)
            ld = int(pos.max()) + 1
            ref = _indexer_ref(_sel(inp.iq, r), _sel(inp.iq_scale, r), _sel(inp.w, r), ik[:ld], iks[:ld], pos, ld)
            m = np.arange(ld)[None, :] <= pos[:, None]
            assert np.array_equal(g_all[r][:, :ld][m], ref[m]), f"E1 scores not bit-exact in rows {b0}.."
            np.testing.assert_array_equal(gi_all[r], oracle.topk(np.where(m, ref, 0.0).astype(np.float32), pos, k,
                                                                 n_threads=oracle_threads()))
        say(f"  E1: all {L} rows: bit-exact scores and indices")
        return
    stats, rel = IndexStats(), RelErr()
    kv_ref = _kv_ref(inp, False)
    for b0 in range(0, L, 1024):
        r = rows[b0:b0 + 1024]
        _verify_prefill_rows(stats, rel, inp, kv_ref, r, g_all[r], gi_all[r], _sel(st.out, r).float().numpy(),
                             _sel(st.lse, r).numpy(), _sel(inp.q, r), k)
        say(f"  rows ..{b0 + len(r)}: out max-abs-rel so far {rel.rel:.3e}")
    say(f"  {stats}")
    say(f"  MLA, all {L} rows: out max-abs-rel {rel.rel:.3e}, lse max abs err {rel.lse:.3e}")
    assert stats.rows == L
    assert rel.rel <= TOL_BF16 and rel.lse <= 2e-2


# ------------------------------------------------------------------ 32K prefill (bench launch)
@pytest.mark.timeout(900)
def test_prefill_32k_bench_launch():
    say("[full C3] 32K prefill as launched by the benchmark")
    cfg, inp, st, kv_slot = bench.setup_prefill_c3(DEV)
    bench.run_prefill_step(cfg, inp, st, kv_slot)
    torch.cuda.synchronize()
    L, k = cfg.L, cfg.k
    rows = _stratified_rows(L, k, MIN_ROWS, seed=3, extra=(4095, 4096, 16383, 16384, 32704, 32705))
    g = _sel(st.scores, rows).numpy()
    gi = _sel(st.idx, rows).numpy()
    stats, rel = IndexStats(), RelErr()
    _verify_prefill_rows(stats, rel, inp, _kv_ref(inp, False), rows, g, gi, _sel(st.out, rows).float().numpy(),
                         _sel(st.lse, rows).numpy(), _sel(inp.q, rows), k)
    # cache contents are the stored tokens, at their shuffled places
    kc = key_cache_rows(st.key_cache, cfg.d_i)[_sel(inp.ik_slot, rows).numpy()]
    assert np.array_equal(kc, u8(_sel(inp.ik, rows)))
    say(f"  {stats}")
    say(f"  MLA, {len(rows)} rows: out max-abs-rel {rel.rel:.3e}, lse max abs err {rel.lse:.3e}")
    assert stats.rows >= MIN_ROWS
    assert rel.rel <= TOL_BF16 and rel.lse <= 2e-2


# ------------------------------------------------------------------ decode (bench launch)
@pytest.mark.timeout(900)
def test_decode_bench_launch():
    import long_context_sparse_fp8_amd as dsa
    say("[full C4] decode, 64 sequences x U[32768, 131072], as launched by the benchmark")
    cfg, inp, caches, newest, ds, kv_slot = bench.setup_decode_c4(DEV)
    bench.run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.synchronize()
    B, k = cfg.decode_batch, cfg.k
    pos = inp.q_pos.cpu().numpy()
    g_all = ds.scores.cpu().numpy()
    gi = ds.idx.cpu().numpy()
    seq_start = inp.seq_start.numpy()
    lens = inp.lens.numpy()
    ld = int(lens.max())
    # indexer rows of every sequence, one oracle call (the rows run in parallel)
    n_keys = int(seq_start[-1] + lens[-1])
    ik, iks = inp.ik[:n_keys].cpu(), inp.ik_scale[:n_keys].cpu()
    iq, iqs, w = inp.iq.cpu(), inp.iq_scale.cpu(), inp.w.cpu()
    ref = oracle.indexer_scores(u8(iq), iqs.numpy(), w.numpy(), u8(ik), iks.numpy(), pos, seq_start=seq_start,
                                q_seq=inp.q_seq.cpu().numpy(), ld=ld, n_threads=oracle_threads())
    stats = IndexStats()
    for b in range(B):
        s0, nb = int(seq_start[b]), int(lens[b])
        A = _abs_scale(iq[b:b + 1], iqs[b:b + 1], w[b:b + 1], ik[s0:s0 + nb], iks[s0:s0 + nb])
        _check_index_rows(stats, g_all[b:b + 1, :nb], ref[b:b + 1, :nb].astype(np.float64), A, pos[b:b + 1], k,
                          gi[b:b + 1])
    say(f"  all {B} sequences: {stats}")
    assert stats.rows == B
    # sparse MLA decode: every query, on the GPU's own indices (only the selected
    # latent rows are copied to the host: the cache is 6 GB)
    packed = np.zeros((B * k, 576), np.uint16)
    new_idx = np.full((B, k), -1, np.int32)
    for b in range(B):
        sel = gi[b][gi[b] >= 0].astype(np.int64) + int(seq_start[b])
        packed[b * k:b * k + len(sel)] = bits16(_sel(inp.kv, sel))
        new_idx[b, :len(sel)] = np.arange(len(sel)) + b * k
    ref_o, ref_l = oracle.sparse_mla(bits16(inp.q), packed, new_idx, SM_SCALE, n_threads=oracle_threads())
    rel = RelErr()
    rel.add(ds.out.float().cpu().numpy(), ref_o, ds.lse.cpu().numpy(), ref_l)
    say(f"  MLA decode, all {B} queries: out max-abs-rel {rel.rel:.3e}, lse max abs err {rel.lse:.3e}")
    assert rel.rel <= TOL_BF16 and rel.lse <= 2e-2
    # the same indices over an FP8 E4M3 latent cache, as the benchmark's FP8 leg launches it
    caches8 = bench.fp8_kv_caches(caches, inp, kv_slot)
    out8, lse8 = torch.empty_like(ds.out), torch.empty_like(ds.lse)
    dsa.sparse_mla_decode(inp.q, caches8.kv_cache, inp.kv_slot_table, inp.q_seq, ds.idx, SM_SCALE, out8, lse8,
                          kv_scale=caches8.kv_scale, n_splits=ds.n_splits, ws=ds.ws)
    torch.cuda.synchronize()
    codes, scales = oracle.kv_quantize(packed)
    ref_o8, ref_l8 = oracle.sparse_mla(bits16(inp.q), codes, new_idx, SM_SCALE, kv_scale=scales,
                                       n_threads=oracle_threads())
    rel8 = RelErr()
    rel8.add(out8.float().cpu().numpy(), ref_o8, lse8.cpu().numpy(), ref_l8)
    say(f"  MLA decode, FP8 latent cache: out max-abs-rel {rel8.rel:.3e}, lse max abs err {rel8.lse:.3e}")
    assert rel8.rel <= TOL_FP8 and rel8.lse <= 2e-2


# ------------------------------------------------------------------ chunked prefill, FP8 KV
@pytest.mark.timeout(900)
def test_chunked_131k_fp8_kv():
    from long_context_sparse_fp8_amd import pipeline as P
    cfg = CONFIGS["C5"]
    L, C, k = cfg.L, cfg.chunk, cfg.k
    n_chunks = L // C
    per_chunk = -(-MIN_ROWS // n_chunks)
    say(f"[full C5] one {L}-token sequence in {C}-token chunks, FP8 latent cache; {per_chunk} rows per chunk")
    inp = synth.make_prefill(cfg, device=DEV, materialize_q=False)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, C, L, k, cfg.h, kv_fp8=True)
    kv_slot = inp.kv_slot_table[0].long()
    rng = np.random.default_rng(5)
    got = []   # (rows, scores, idx, out, lse, q)
    for c0 in range(0, L, C):
        c1 = c0 + C
        P.store_tokens(st, inp.ik[c0:c1], inp.ik_scale[c0:c1], inp.ik_slot[c0:c1], inp.kv[c0:c1], kv_slot[c0:c1])
        q = inp.q_chunk(c0, c1)
        P.prefill_step(st, inp.iq[c0:c1], inp.iq_scale[c0:c1], inp.w[c0:c1], inp.page_table, inp.kv_slot_table,
                       inp.q_seq[c0:c1], inp.q_pos[c0:c1], q, k, SM_SCALE)
        loc = {0, 1, C - 2, C - 1}                                            # chunk boundaries
        if c0 == 0:
            loc |= {2, k - 1, k, k + 1} | set(rng.integers(0, k, 6).tolist())   # fewer candidates than k
        while len(loc) < per_chunk:
            loc |= set(rng.integers(0, C, per_chunk - len(loc)).tolist())
        loc = np.array(sorted(loc))
        got.append((c0 + loc, _sel(st.scores, loc).numpy(), _sel(st.idx, loc).numpy(),
                    _sel(st.out, loc).float().numpy(), _sel(st.lse, loc).numpy(), _sel(q, loc)))
        torch.cuda.synchronize()
        del q
    say(f"  ran {n_chunks} chunks")
    # FP8 cache bytes equal the oracle's quantizer on every stored row
    kv_ref = _kv_ref(inp, True)
    slot_np = kv_slot.cpu().numpy()
    assert np.array_equal(u8(st.kv_cache)[slot_np], kv_ref[0])
    assert np.array_equal(st.kv_scale.cpu().numpy()[slot_np], kv_ref[1])
    stats, rel = IndexStats(), RelErr()
    for rows, g, gi, go, gl, q in got:
        _verify_prefill_rows(stats, rel, inp, kv_ref, rows, g, gi, go, gl, q, k)
    say(f"  {stats}")
    say(f"  MLA (FP8 KV), {stats.rows} rows: out max-abs-rel {rel.rel:.3e}, lse max abs err {rel.lse:.3e}")
    assert stats.rows >= MIN_ROWS
    assert rel.rel <= TOL_FP8 and rel.lse <= 2e-2
