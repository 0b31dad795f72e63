"""GPU parity at the full workload sizes, on sampled rows the oracle computes one
by one.

Each workload runs exactly as the benchmark launches it (same input
generation, same calls, same launch geometry):
  * 8K prefill  (B=1, L=8192, k=2048, 64x128 FP8 indexer, 128-head MLA),
    plus the same shape in the exact-arithmetic regime E1;
  * 32K prefill (L=32768, shuffled 64-token pages and KV slots);
  * decode      (64 sequences, contexts ~ U[32768, 131072], one query each);
  * chunked prefill of one 131072-token sequence in 8192-token chunks with
    an FP8 (E4M3 + per-token scale) latent cache.
Rows are verified completely (whole indexer row, its top-k, its MLA output)
on a stratified sample: the first rows, rows around k, chunk boundaries, the
last rows and uniform picks.  Top-k is checked bit-exactly from the GPU's own
scores on every sampled row (all rows for 8K and decode); end-to-end indices
are checked against the oracle's own scores up to near-ties inside the
a-priori FP8-MFMA error bound.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from synth.configs import CONFIGS, SM_SCALE, Config
from gpu_common import DEV, say, bits16, u8, max_abs_rel, oracle_threads, key_cache_rows
import long_context_sparse_fp8_amd as dsa
from long_context_sparse_fp8_amd import pipeline as P

pytestmark = pytest.mark.gpu

BOUND_C = 2.0 ** -9
TOL_BF16, TOL_FP8 = 2e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dsa.lib()
    yield
    torch.cuda.empty_cache()


def _rows(L, k, extra=(), n_uniform=24, seed=0):
    rng = np.random.default_rng(seed)
    r = [0, 1, 2, k - 2, k - 1, k, k + 1, L - 2, L - 1, *extra]
    r += list(rng.integers(0, L, n_uniform))
    r = np.unique(np.array([x for x in r if 0 <= x < L], dtype=np.int64))
    return r


def _abs_scale(iq, iqs, w, ik, iks):
    """A[r, s] = qs_r ks_s sum_j |w_rj| sum_i |q_rji k_si| (float64, host tensors)."""
    qv = np.abs(torch.from_numpy(u8(iq)).view(torch.float8_e4m3fn).double().numpy())   # [r, H, D]
    kv = np.abs(torch.from_numpy(u8(ik)).view(torch.float8_e4m3fn).double().numpy())   # [N, D]
    v = np.einsum("rh,rhd->rd", np.abs(w.double().numpy()), qv)
    return (v @ kv.T) * iqs.double().numpy()[:, None] * iks.double().numpy()[None, :]


def _check_index_rows(g_scores, ref_scores, A, pos, k, g_idx):
    """g_scores / ref_scores / A: [r, >= pos+1] for the sampled rows; g_idx [r, k].
    1) top-k on the GPU's scores is bit-exact (oracle.topk on identical inputs);
    2) GPU scores are within BOUND_C * A of the exact scores;
    3) end-to-end indices differ from the oracle's only at near-ties.
    Returns (max error ratio, number of index mismatches)."""
    ld = g_scores.shape[1]
    mask = np.arange(ld)[None, :] <= pos[:, None]
    np.testing.assert_array_equal(g_idx, oracle.topk(np.where(mask, g_scores, 0.0).astype(np.float32), pos, k,
                                                     n_threads=oracle_threads()))
    err = np.abs(g_scores.astype(np.float64) - ref_scores)[mask]
    delta = BOUND_C * A[mask] + 1e-30
    ratio = float((err / delta).max())
    assert ratio <= 1.0, f"indexer error {ratio:.3f} x the bound"
    r_idx = oracle.topk(np.where(mask, ref_scores, 0.0).astype(np.float32), pos, k, n_threads=oracle_threads())
    mism = 0
    for r in range(len(pos)):
        G = set(g_idx[r][g_idx[r] >= 0].tolist())
        R = set(r_idx[r][r_idx[r] >= 0].tolist())
        if G == R:
            continue
        gr, rg = np.array(sorted(G - R)), np.array(sorted(R - G))
        assert len(gr) == len(rg)
        mism += len(gr)
        d = BOUND_C * A[r]
        # every swapped pair must be a near-tie: the GPU could rank s above r only if
        # their exact scores are within the two error bounds of each other
        lo_r = (ref_scores[r, rg] - d[rg]).min()
        hi_s = (ref_scores[r, gr] + d[gr]).max()
        assert (ref_scores[r, gr] + d[gr] >= lo_r).all() and (ref_scores[r, rg] - d[rg] <= hi_s).all(), \
            f"row {r}: index swap that is not a near-tie"
    return ratio, mism


def _mla_rows_ref(q_rows_bits, kv_logical, idx_rows, kv_scale=None, seq_start=None, q_seq=None):
    """Oracle MLA for a few rows, handing it only the rows each query selected:
    row r's selected logical rows are packed at [r * k, r * k + n_r)."""
    n, k = idx_rows.shape
    rows, new_idx = [], np.full((n, k), -1, np.int32)
    for r in range(n):
        sel = idx_rows[r][idx_rows[r] >= 0]
        base = 0 if seq_start is None else int(seq_start[q_seq[r]])
        rows.append(sel.astype(np.int64) + base)
        new_idx[r, :len(sel)] = np.arange(len(sel)) + r * k
    width = kv_logical.shape[1]
    packed = np.zeros((n * k, width), dtype=kv_logical.dtype)
    packed_scale = np.zeros(n * k, np.float32) if kv_scale is not None else None
    for r in range(n):
        m = len(rows[r])
        packed[r * k:r * k + m] = kv_logical[rows[r]]
        if kv_scale is not None:
            packed_scale[r * k:r * k + m] = kv_scale[rows[r]]
    # every row is "sequence 0" of the packed array; new_idx are absolute packed rows
    return oracle.sparse_mla(q_rows_bits, packed, new_idx, SM_SCALE, kv_scale=packed_scale,
                             n_threads=oracle_threads())


def _sel(t, rows):
    """Rows of a (device) tensor picked by a numpy index array, copied to the host."""
    return t[torch.as_tensor(np.asarray(rows), device=t.device)].cpu()


def _indexer_ref(inp_iq, inp_iqs, inp_w, ik, iks, pos):
    return oracle.indexer_scores(u8(inp_iq), inp_iqs.numpy(), inp_w.numpy(), u8(ik), iks.numpy(), pos,
                                 ld=int(pos.max()) + 1, n_threads=oracle_threads())


# ------------------------------------------------------------------ 8K prefill
@pytest.mark.parametrize("exact", [False, True])
def test_prefill_8k_full(exact):
    cfg = CONFIGS["C2"]
    say(f"[full C2] L={cfg.L} k={cfg.k} exact={exact}")
    inp = synth.make_prefill(cfg, device=DEV, exact=exact)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, cfg.L, cfg.L, cfg.k, cfg.h)
    P.store_tokens(st, inp.ik, inp.ik_scale, inp.ik_slot, inp.kv, inp.kv_slot_table[0].long())
    P.prefill_step(st, inp.iq, inp.iq_scale, inp.w, inp.page_table, inp.kv_slot_table, inp.q_seq, inp.q_pos,
                   inp.q, cfg.k, SM_SCALE)
    torch.cuda.synchronize()
    L, k = cfg.L, cfg.k
    pos_all = np.arange(L, dtype=np.int32)
    g_all = st.scores.cpu().numpy()
    gi_all = st.idx.cpu().numpy()
    # top-k of every row from the GPU's own scores: bit-exact
    mask = np.arange(L)[None, :] <= pos_all[:, None]
    np.testing.assert_array_equal(gi_all, oracle.topk(np.where(mask, g_all, 0.0).astype(np.float32), pos_all, k,
                                                      n_threads=oracle_threads()))
    say("  top-k of all 8192 rows bit-exact from identical scores")
    rows = _rows(L, k, n_uniform=40, seed=2 + exact)
    pos = pos_all[rows]
    iq, iqs, w = _sel(inp.iq, rows), _sel(inp.iq_scale, rows), _sel(inp.w, rows)
    ik, iks = inp.ik.cpu(), inp.ik_scale.cpu()
    ref = _indexer_ref(iq, iqs, w, ik, iks, pos)
    g = g_all[rows][:, :ref.shape[1]]
    if exact:
        m = np.arange(ref.shape[1])[None, :] <= pos[:, None]
        assert np.array_equal(g[m], ref[m]), "E1 scores are not bit-exact"
        r_idx = oracle.topk(np.where(m, ref, 0.0).astype(np.float32), pos, k, n_threads=oracle_threads())
        np.testing.assert_array_equal(gi_all[rows], r_idx)
        say(f"  E1: {len(rows)} rows bit-exact scores and indices")
    else:
        A = _abs_scale(iq, iqs, w, ik, iks)
        ratio, mism = _check_index_rows(g, ref.astype(np.float64), A, pos, k, gi_all[rows])
        say(f"  indexer err/bound max {ratio:.4f}; end-to-end index mismatches (near-ties) {mism}")
    mrows = rows[:: max(1, len(rows) // 24)]
    ref_o, ref_l = _mla_rows_ref(bits16(_sel(inp.q, mrows)), bits16(inp.kv), gi_all[mrows])
    e = max_abs_rel(_sel(st.out, mrows).float().numpy(), ref_o)
    el = float(np.abs(_sel(st.lse, mrows).numpy() - ref_l).max())
    say(f"  MLA {len(mrows)} rows: out max-abs-rel {e:.3e}, lse max abs err {el:.3e}")
    assert e <= TOL_BF16 and el <= 2e-2


# ------------------------------------------------------------------ 32K prefill (bench launch)
def test_prefill_32k_bench_launch():
    say("[full C3] 32K prefill as launched by the benchmark")
    cfg, inp, st, kv_slot = bench.setup_prefill_c3(DEV)
    bench.run_prefill_step(cfg, inp, st, kv_slot)
    torch.cuda.synchronize()
    L, k = cfg.L, cfg.k
    rows = _rows(L, k, extra=(4095, 4096, 16383, 16384, 32704, 32705), n_uniform=22, seed=3)
    pos = rows.astype(np.int32)
    iq, iqs, w = _sel(inp.iq, rows), _sel(inp.iq_scale, rows), _sel(inp.w, rows)
    ik, iks = inp.ik.cpu(), inp.ik_scale.cpu()
    ref = _indexer_ref(iq, iqs, w, ik, iks, pos)
    g = _sel(st.scores, rows).numpy()[:, :ref.shape[1]]
    gi = _sel(st.idx, rows).numpy()
    A = _abs_scale(iq, iqs, w, ik, iks)
    ratio, mism = _check_index_rows(g, ref.astype(np.float64), A, pos, k, gi)
    say(f"  {len(rows)} rows: indexer err/bound max {ratio:.4f}; index mismatches (near-ties) {mism}")
    # cache contents are the stored tokens, at their shuffled places
    kc = key_cache_rows(st.key_cache, cfg.d_i)[_sel(inp.ik_slot, rows).numpy()]
    assert np.array_equal(kc, u8(_sel(inp.ik, rows)))
    ref_o, ref_l = _mla_rows_ref(bits16(_sel(inp.q, rows)), bits16(inp.kv), gi)
    e = max_abs_rel(_sel(st.out, rows).float().numpy(), ref_o)
    el = float(np.abs(_sel(st.lse, rows).numpy() - ref_l).max())
    say(f"  MLA: out max-abs-rel {e:.3e}, lse max abs err {el:.3e}")
    assert e <= TOL_BF16 and el <= 2e-2


# ------------------------------------------------------------------ decode (bench launch)
def test_decode_bench_launch():
    say("[full C4] decode, 64 sequences x U[32768, 131072], as launched by the benchmark")
    cfg, inp, caches, newest, ds, kv_slot = bench.setup_decode_c4(DEV)
    bench.run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.synchronize()
    B, k = cfg.decode_batch, cfg.k
    pos = inp.q_pos.cpu().numpy()
    g_all = ds.scores.cpu().numpy()
    gi = ds.idx.cpu().numpy()
    ld = g_all.shape[1]
    mask = np.arange(ld)[None, :] <= pos[:, None]
    np.testing.assert_array_equal(gi, oracle.topk(np.where(mask, g_all, 0.0).astype(np.float32), pos, k,
                                                  n_threads=oracle_threads()))
    say("  top-k of all 64 rows bit-exact from identical scores")
    seq_start = inp.seq_start.numpy()
    lens = inp.lens.numpy()
    sample = np.unique(np.concatenate([[int(np.argmin(lens)), int(np.argmax(lens))],
                                       np.random.default_rng(4).choice(B, 6, replace=False)]))
    tot_mism = 0
    for b in sample:
        s0, nb = int(seq_start[b]), int(lens[b])
        iq, iqs, w = inp.iq[b:b + 1].cpu(), inp.iq_scale[b:b + 1].cpu(), inp.w[b:b + 1].cpu()
        ik, iks = inp.ik[s0:s0 + nb].cpu(), inp.ik_scale[s0:s0 + nb].cpu()
        p = pos[b:b + 1]
        ref = _indexer_ref(iq, iqs, w, ik, iks, p)
        A = _abs_scale(iq, iqs, w, ik, iks)
        ratio, mism = _check_index_rows(g_all[b:b + 1, :nb], ref.astype(np.float64), A, p, k, gi[b:b + 1])
        tot_mism += mism
        say(f"  seq {b} (N={nb}): indexer err/bound max {ratio:.4f}, index mismatches {mism}")
    # sparse MLA decode: every query, on the GPU's own indices
    kv_rows = []
    for b in range(B):
        sel = gi[b][gi[b] >= 0].astype(np.int64) + int(seq_start[b])
        kv_rows.append(sel)
    packed = bits16(_sel(inp.kv, np.concatenate(kv_rows)))
    packed_full = np.zeros((B * k, 576), np.uint16)
    new_idx = np.full((B, k), -1, np.int32)
    o = 0
    for b in range(B):
        m = len(kv_rows[b])
        packed_full[b * k:b * k + m] = packed[o:o + m]
        new_idx[b, :m] = np.arange(m) + b * k
        o += m
    ref_o, ref_l = oracle.sparse_mla(bits16(inp.q), packed_full, new_idx, SM_SCALE, n_threads=oracle_threads())
    e = max_abs_rel(ds.out.float().cpu().numpy(), ref_o)
    el = float(np.abs(ds.lse.cpu().numpy() - ref_l).max())
    say(f"  MLA decode, all 64 queries: out max-abs-rel {e:.3e}, lse max abs err {el:.3e}")
    assert e <= TOL_BF16 and el <= 2e-2
    # the same indices over an FP8 E4M3 latent cache, as the benchmark's FP8 leg launches it
    caches8 = bench.fp8_kv_caches(caches, inp, kv_slot)
    out8, lse8 = torch.empty_like(ds.out), torch.empty_like(ds.lse)
    dsa.sparse_mla_decode(inp.q, caches8.kv_cache, inp.kv_slot_table, inp.q_seq, ds.idx, SM_SCALE, out8, lse8,
                          kv_scale=caches8.kv_scale, n_splits=ds.n_splits, ws=ds.ws)
    torch.cuda.synchronize()
    codes, scales = oracle.kv_quantize(packed_full)
    ref_o8, ref_l8 = oracle.sparse_mla(bits16(inp.q), codes, new_idx, SM_SCALE, kv_scale=scales,
                                       n_threads=oracle_threads())
    e8 = max_abs_rel(out8.float().cpu().numpy(), ref_o8)
    el8 = float(np.abs(lse8.cpu().numpy() - ref_l8).max())
    say(f"  MLA decode, FP8 latent cache: out max-abs-rel {e8:.3e}, lse max abs err {el8:.3e}")
    assert e8 <= TOL_FP8 and el8 <= 2e-2


# ------------------------------------------------------------------ chunked prefill, FP8 KV
def test_chunked_131k_fp8_kv():
    cfg = CONFIGS["C5"]
    L, C, k = cfg.L, cfg.chunk, cfg.k
    say(f"[full C5] one {L}-token sequence in {C}-token chunks, FP8 latent cache")
    inp = synth.make_prefill(cfg, device=DEV, materialize_q=False)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, C, L, k, cfg.h, kv_fp8=True)
    kv_slot = inp.kv_slot_table[0].long()
    rng = np.random.default_rng(5)
    checks = []   # (chunk start, local rows)
    for c0 in range(0, L, C):
        c1 = c0 + C
        P.store_tokens(st, inp.ik[c0:c1], inp.ik_scale[c0:c1], inp.ik_slot[c0:c1], inp.kv[c0:c1], kv_slot[c0:c1])
        P.prefill_step(st, inp.iq[c0:c1], inp.iq_scale[c0:c1], inp.w[c0:c1], inp.page_table, inp.kv_slot_table,
                       inp.q_seq[c0:c1], inp.q_pos[c0:c1], inp.q_chunk(c0, c1), k, SM_SCALE)
        loc = np.unique(np.concatenate([[0, C - 1], rng.integers(0, C, 1)]))
        if c0 == 0:
            loc = np.unique(np.concatenate([loc, [1, k - 1, k, k + 1]]))
        rows = c0 + loc
        checks.append((rows, _sel(st.scores, loc).numpy(), _sel(st.idx, loc).numpy(),
                       _sel(st.out, loc).float().numpy(), _sel(st.lse, loc).numpy()))
        torch.cuda.synchronize()
    say(f"  ran {L // C} chunks")
    # FP8 cache bytes equal the oracle's quantizer on every stored row
    codes, scales = oracle.kv_quantize(bits16(inp.kv))
    slot_np = kv_slot.cpu().numpy()
    assert np.array_equal(u8(st.kv_cache)[slot_np], codes)
    assert np.array_equal(st.kv_scale.cpu().numpy()[slot_np], scales)
    rows = np.concatenate([c[0] for c in checks])
    g = np.concatenate([c[1] for c in checks])
    gi = np.concatenate([c[2] for c in checks])
    go = np.concatenate([c[3] for c in checks])
    gl = np.concatenate([c[4] for c in checks])
    pos = rows.astype(np.int32)
    iq, iqs, w = _sel(inp.iq, rows), _sel(inp.iq_scale, rows), _sel(inp.w, rows)
    ik, iks = inp.ik.cpu(), inp.ik_scale.cpu()
    ref = _indexer_ref(iq, iqs, w, ik, iks, pos)
    A = _abs_scale(iq, iqs, w, ik, iks)
    ratio, mism = _check_index_rows(g[:, :ref.shape[1]], ref.astype(np.float64), A, pos, k, gi)
    say(f"  {len(rows)} rows: indexer err/bound max {ratio:.4f}; index mismatches (near-ties) {mism}")
    qrows = torch.cat([inp.q_chunk(int(r), int(r) + 1) for r in rows])
    ref_o, ref_l = _mla_rows_ref(bits16(qrows), codes, gi, kv_scale=scales)
    e = max_abs_rel(go, ref_o)
    el = float(np.abs(gl - ref_l).max())
    say(f"  MLA (FP8 KV): out max-abs-rel {e:.3e}, lse max abs err {el:.3e}")
    assert e <= TOL_FP8 and el <= 2e-2
