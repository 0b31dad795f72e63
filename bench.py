"""Benchmark of the DSA hot path on one MI355X.

Headline step (value): one prefill pass over a 32768-token sequence (B=1,
causal, k=2048; indexer 64 heads x 128 FP8 keys in 64-token pages with a
shuffled page table; MLA 128 heads, 576/512-d bf16 latent rows in a
token-granular cache with shuffled slots):
    cache stores -> indexer scores -> top-k -> sparse MLA prefill
reported as prefill tokens/s.  Second figure: one decode step for 64
sequences with contexts drawn uniformly from [32768, 131072] (one query
each): cache stores -> indexer + top-k (the fused call) -> sparse MLA
decode, in us/step, and the same step with the indexer and top-k as two calls.

All inputs are seeded synthetic tensors generated on the GPU before timing.
The timed steps run without instrumentation; a second pass of the same steps
brackets each stage by HIP events on the stream the kernels run on, and the
roofline object uses the algorithmic work per launch divided by that average
launch time.  The CPU baseline runs the oracle (the plain
double-precision C reference) on a bounded sample of query rows of the same
workload.

HBM traffic of the dominant kernel comes from rocprofv3 counter runs
(FETCH_SIZE, WRITE_SIZE) recorded in profiles/hbm_traffic.txt together with
the SHA-256 of the kernel's sources; it is reported only while those sources
are unchanged, otherwise as null.  --calib-copy adds one plain 1 GiB
device-to-device copy after the timed work, the known-size kernel those
counter runs are scaled by.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--calib-copy] [--configs]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from synth.configs import CONFIGS, SM_SCALE  # noqa: E402
import long_context_sparse_fp8_amd as dsa  # noqa: E402
from long_context_sparse_fp8_amd import pipeline as P  # noqa: E402

METRIC = "DSA prefill tokens/s at 32K & decode us/step at 128K ctx; % MFMA/HBM roofline"
PEAK_FP8 = 5000.0      # TFLOP/s, dense MFMA (MI355X datasheet)
PEAK_BF16 = 2500.0
PEAK_HBM = 8000.0      # GB/s


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic.txt, or None when
    nothing is recorded or a source it was measured on has changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if not line.startswith("kernel="):
            continue
        f = dict(kv.split("=", 1) for kv in line.split())
        if f.get("kernel") != kernel:
            continue
        for src, digest in zip(f["sources"].split(","), f["sha256"].split(",")):
            path = os.path.join(ROOT, src)
            if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest()[:16] != digest:
                return None
        return float(f["traffic_bytes"])
    return None


def calib_copy(dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size for scaling the HBM counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {reps} x {nbytes} bytes")


def measured_copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Bytes moved (read + write) per second by a plain 1 GiB device-to-device
    copy: the HBM bandwidth a streaming kernel reaches on this machine, beside the
    8 TB/s datasheet peak the roofline fractions use."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def measured_bf16_gemm(dev, n=8192, reps=10):
    """TFLOP/s of torch's dense bf16 matmul (the vendor GEMM) at n x n x n: what a
    library GEMM reaches on this machine, beside the 2.5 PFLOP/s datasheet peak."""
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del c
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def measured_fp8_gemm(dev, n=8192, reps=10):
    """TFLOP/s of torch's FP8 (E4M3) scaled matmul at n x n x n, or None where
    this torch build has no FP8 GEMM for the device."""
    try:
        a = torch.randn((n, n), device=dev).to(torch.float8_e4m3fn)
        b = torch.randn((n, n), device=dev).to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=dev)
        mm = lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        mm()
        torch.cuda.synchronize()
    except (RuntimeError, TypeError, AttributeError):
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mm()
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class StageTimer:
    """Per-stage HIP events on the current stream; averages over the timed steps."""

    def __init__(self, names):
        self.names = names
        self.ev = {n: [] for n in names}

    def mark(self, name):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        self.ev[name].append((s, e))
        return e

    def avg_ms(self):
        torch.cuda.synchronize()
        return {n: float(np.mean([s.elapsed_time(e) for s, e in v])) if v else 0.0 for n, v in self.ev.items()}


# ---------------------------------------------------------------------------- prefill
def prefill_work(L, k, h_i, d_i, h):
    pairs = L * (L + 1) // 2
    sel = sum(min(k, t + 1) for t in range(L))
    return {
        "indexer_flops": 2.0 * h_i * d_i * pairs,
        "mla_flops": 2.0 * h * (576 + 512) * sel,
        "topk_bytes": 4.0 * sum(t + 1 for t in range(L) if t + 1 > k) + 4.0 * L * k,
        "selected_pairs": sel,
        "pairs": pairs,
    }


def setup_prefill_c3(dev):
    cfg = CONFIGS["C3"]
    inp = synth.make_prefill(cfg, device=dev)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, cfg.L, cfg.L, cfg.k, cfg.h, device=dev)
    kv_slot = inp.kv_slot_table[0].long()
    return cfg, inp, st, kv_slot


def run_prefill_step(cfg, inp, st, kv_slot, timer=None):
    def t(name):
        return timer.mark(name) if timer else None

    e = t("store")
    P.store_tokens(st, inp.ik, inp.ik_scale, inp.ik_slot, inp.kv, kv_slot)
    if e: e.record()
    e = t("indexer")
    dsa.indexer_scores(inp.iq, inp.iq_scale, inp.w, st.key_cache, st.key_scale, inp.page_table, inp.q_seq,
                       inp.q_pos, st.scores)
    if e: e.record()
    e = t("topk")
    dsa.topk(st.scores, inp.q_pos, cfg.k, st.idx)
    if e: e.record()
    e = t("mla")
    dsa.sparse_mla_prefill(inp.q, st.kv_cache, inp.kv_slot_table, inp.q_seq, st.idx, SM_SCALE, st.out, st.lse)
    if e: e.record()


# ---------------------------------------------------------------------------- decode
def setup_decode_c4(dev):
    cfg = CONFIGS["C4"]
    inp = synth.make_decode(cfg, device=dev)
    caches = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, 1, 1, cfg.k, cfg.h, device=dev)
    kv_slot = torch.empty(inp.n_slots, dtype=torch.int64)
    kvt = inp.kv_slot_table.cpu()
    for b in range(cfg.decode_batch):
        s0, nb = int(inp.seq_start[b]), int(inp.lens[b])
        kv_slot[s0:s0 + nb] = kvt[b, :nb].long()
    kv_slot = kv_slot.to(dev)
    P.store_tokens(caches, inp.ik, inp.ik_scale, inp.ik_slot, inp.kv, kv_slot)
    # the step stores each sequence's newest token (its query position) again
    last = (inp.seq_start + inp.lens - 1).to(dev)
    newest = dict(ik=inp.ik[last], ik_scale=inp.ik_scale[last], ik_slot=inp.ik_slot[last], kv=inp.kv[last],
                  kv_slot=kv_slot[last])
    ld = int(inp.lens.max())
    ds = P.alloc_decode(cfg.decode_batch, ld, cfg.k, cfg.h, device=dev)
    torch.cuda.synchronize()
    return cfg, inp, caches, newest, ds, kv_slot


def fp8_kv_caches(caches, inp, kv_slot):
    """The same caches with the latent rows quantized to FP8 E4M3 + a per-token scale."""
    kv8 = torch.zeros((inp.n_slots, 576), dtype=torch.uint8, device=caches.kv_cache.device)
    sc8 = torch.zeros(inp.n_slots, dtype=torch.float32, device=caches.kv_cache.device)
    dsa.kv_cache_store(inp.kv, kv_slot, kv8, sc8)
    torch.cuda.synchronize()
    return dataclasses.replace(caches, kv_cache=kv8, kv_scale=sc8)


def run_decode_step(cfg, inp, caches, newest, ds, timer=None):
    def t(name):
        return timer.mark(name) if timer else None

    e = t("store")
    P.store_tokens(caches, newest["ik"], newest["ik_scale"], newest["ik_slot"], newest["kv"], newest["kv_slot"])
    if e: e.record()
    if ds.fused_ws is not None:            # fused indexer -> top-k: one call, one stage
        e = t("indexer_topk")
        dsa.indexer_topk(inp.iq, inp.iq_scale, inp.w, caches.key_cache, caches.key_scale, inp.page_table, inp.q_seq,
                         inp.q_pos, ds.scores, cfg.k, ds.idx, ds.fused_ws)
        if e: e.record()
    else:
        e = t("indexer")
        dsa.indexer_scores(inp.iq, inp.iq_scale, inp.w, caches.key_cache, caches.key_scale, inp.page_table,
                           inp.q_seq, inp.q_pos, ds.scores)
        if e: e.record()
        e = t("topk")
        dsa.topk(ds.scores, inp.q_pos, cfg.k, ds.idx, ws=ds.topk_ws)
        if e: e.record()
    e = t("mla")
    dsa.sparse_mla_decode(inp.q, caches.kv_cache, inp.kv_slot_table, inp.q_seq, ds.idx, SM_SCALE, ds.out, ds.lse,
                          kv_scale=caches.kv_scale, n_splits=ds.n_splits, ws=ds.ws)
    if e: e.record()


def decode_kernels(db, stages, mla_traffic_key="sparse_mla_decode"):
    """Achieved HBM rate of each decode stage from its algorithmic bytes (a fused
    indexer -> top-k stage carries the bytes of both), with the recorded HBM
    traffic of the 64-query launches where it applies."""
    parts = ([("indexer_topk", db["indexer_bytes"] + db["topk_bytes"], "indexer_topk")] if "indexer_topk" in stages
             else [("indexer", db["indexer_bytes"], "indexer"), ("topk", db["topk_bytes"], "topk")])
    parts.append(("sparse_mla_decode", db["mla_bytes"], "mla"))
    out = {}
    for name, nbytes, st in parts:
        gbs = nbytes / (stages[st] * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s", "us": stages[st] * 1e3,
                     "frac": gbs / PEAK_HBM}
    # HBM bytes per launch from the recorded counter runs (null when not recorded for these sources)
    if "indexer_topk" in out:
        parts = [recorded_traffic(n) for n in ("indexer_decode", "topk_fused_part", "topk_fused_merge")]
        out["indexer_topk"]["traffic"] = None if None in parts else sum(parts)
    out["sparse_mla_decode"]["traffic"] = recorded_traffic(mla_traffic_key) if mla_traffic_key else None
    return out


def time_decode(args, cfg, inp, caches, newest, ds):
    """Warm-up, then `args.steps` timed decode steps: (seconds per step, stage ms).
    The timed steps carry no instrumentation (events between a step's launches
    cost the GPU ≈ 20 us per step at this size); the stage times come from a
    second pass of the same steps with events."""
    for _ in range(args.warmup):
        run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    timer = StageTimer(["store", "indexer_topk", "mla"] if ds.fused_ws is not None else
                       ["store", "indexer", "topk", "mla"])
    for _ in range(args.steps):
        run_decode_step(cfg, inp, caches, newest, ds, timer)
    torch.cuda.synchronize()
    return wall, timer.avg_ms()


def time_decode_graph(args, cfg, inp, caches, newest, ds):
    """The decode step captured once as a HIP graph (the 7 launches of the step in
    one submission, as a serving loop would run it) and replayed: (seconds per
    step, whether the replayed outputs equal the eager ones bit for bit)."""
    run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.synchronize()
    ref = (ds.idx.clone(), ds.out.clone(), ds.lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_decode_step(cfg, inp, caches, newest, ds)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_decode_step(cfg, inp, caches, newest, ds)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, (ds.idx, ds.out, ds.lse)))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    del graph
    return wall, same


def decode_bytes(inp, k, h, kv_row_bytes=1152):
    """Algorithmic HBM bytes per decode step; a latent row is 1152 B in bf16,
    576 B of codes + a 4-byte scale in FP8.  With several queries per sequence
    the keys of a sequence count once (the scan they could share)."""
    n_keys = int(inp.lens.sum())
    n_q = int(inp.q_pos.numel())
    n_scores = float((inp.q_pos.long() + 1).sum())
    return {
        "indexer_bytes": n_keys * (128 + 4) + inp.iq.numel() + 4.0 * n_scores,   # keys + scales read, scores written
        "topk_bytes": 4.0 * n_scores + 4.0 * n_q * k,
        "mla_bytes": n_q * k * (kv_row_bytes + 4 + 4) + inp.q.numel() * 2 + n_q * h * 512 * 2,
    }


# ---------------------------------------------------------------------------- CPU baseline
def cpu_model():
    """The host CPU's model name (first /proc/cpuinfo entry), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rows(inp, cfg, rows, threads):
    """Seconds the oracle takes for the full indexer row, top-k and sparse MLA of each row."""
    import oracle
    u8 = lambda t: t.detach().cpu().contiguous().numpy().view(np.uint8)
    b16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    iq, iqs, w = u8(inp.iq[rows]), inp.iq_scale[rows].cpu().numpy(), inp.w[rows].cpu().numpy()
    ik, iks = u8(inp.ik), inp.ik_scale.cpu().numpy()
    q, kv = b16(inp.q[rows]), b16(inp.kv)
    pos = rows.astype(np.int32)
    t0 = time.perf_counter()
    sc = oracle.indexer_scores(iq, iqs, w, ik, iks, pos, ld=cfg.L, n_threads=threads)
    idx = oracle.topk(sc, pos, cfg.k, n_threads=threads)
    oracle.sparse_mla(q, kv, idx, SM_SCALE, n_threads=threads)
    return time.perf_counter() - t0


def cpu_baseline(inp, cfg, n_rows, n_rows_single=48):
    """The oracle on the host cores: all threads over n_rows evenly spaced query
    rows of the 32K prefill, and one thread over n_rows_single of them."""
    threads = os.cpu_count() or 1
    rows = np.linspace(0, cfg.L - 1, n_rows).round().astype(np.int64)
    dt = _oracle_rows(inp, cfg, rows, threads)
    rows1 = np.linspace(0, cfg.L - 1, n_rows_single).round().astype(np.int64)
    dt1 = _oracle_rows(inp, cfg, rows1, 1)
    return {"value": n_rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} evenly spaced query rows of the 32K prefill (positions 0..{cfg.L - 1}), full "
                      f"indexer row + top-k + sparse MLA each, {dt:.1f} s wall on {threads} threads",
            "single_thread": {"value": n_rows_single / dt1, "unit": "tokens/s", "seconds": dt1,
                              "sample": f"{n_rows_single} evenly spaced rows of the same prefill on 1 thread"},
            "cpu_model": cpu_model()}


# ---------------------------------------------------------------------------- all configs
def oracle_prefill_rate(inp, cfg, rows, ld):
    """Oracle tokens/s over the given query rows of a prefill input (full indexer
    row + top-k + sparse MLA each)."""
    import oracle
    u8 = lambda t: t.detach().cpu().contiguous().numpy().view(np.uint8)
    b16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    rows = np.asarray(rows, dtype=np.int64)
    iq, iqs, w = u8(inp.iq[rows]), inp.iq_scale[rows].cpu().numpy(), inp.w[rows].cpu().numpy()
    ik, iks = u8(inp.ik), inp.ik_scale.cpu().numpy()
    q = inp.q[rows] if inp.q is not None else torch.cat([inp.q_chunk(int(r), int(r) + 1) for r in rows])
    kv = b16(inp.kv)
    pos = inp.q_pos[rows].cpu().numpy().astype(np.int32)
    threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    sc = oracle.indexer_scores(iq, iqs, w, ik, iks, pos, ld=ld, n_threads=threads)
    idx = oracle.topk(sc, pos, cfg.k, n_threads=threads)
    if cfg.kv_fp8:
        codes, scales = oracle.kv_quantize(kv)
        oracle.sparse_mla(b16(q), codes, idx, SM_SCALE, kv_scale=scales, n_threads=threads)
    else:
        oracle.sparse_mla(b16(q), kv, idx, SM_SCALE, n_threads=threads)
    dt = time.perf_counter() - t0
    return {"tokens_per_s": len(rows) / dt, "rows": int(len(rows)), "seconds": dt, "cores": threads}


def oracle_decode_rate(inp, cfg, n_seq):
    """Oracle time of one decode query (indexer over its whole context, top-k,
    sparse MLA) on the first n_seq sequences, scaled to a step of all of them."""
    import oracle
    u8 = lambda t: t.detach().cpu().contiguous().numpy().view(np.uint8)
    b16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    n_keys = int(inp.lens[:n_seq].sum())
    pos = inp.q_pos[:n_seq].cpu().numpy().astype(np.int32)
    seq_start = inp.seq_start[:n_seq].numpy()
    q_seq = inp.q_seq[:n_seq].cpu().numpy()
    threads = os.cpu_count() or 1
    ik, iks, kv = u8(inp.ik[:n_keys]), inp.ik_scale[:n_keys].cpu().numpy(), b16(inp.kv[:n_keys])
    t0 = time.perf_counter()
    sc = oracle.indexer_scores(u8(inp.iq[:n_seq]), inp.iq_scale[:n_seq].cpu().numpy(), inp.w[:n_seq].cpu().numpy(),
                               ik, iks, pos, seq_start=seq_start, q_seq=q_seq, ld=int(inp.lens.max()),
                               n_threads=threads)
    idx = oracle.topk(sc, pos, cfg.k, n_threads=threads)
    oracle.sparse_mla(b16(inp.q[:n_seq]), kv, idx, SM_SCALE, seq_start=seq_start, q_seq=q_seq, n_threads=threads)
    dt = time.perf_counter() - t0
    n_all = int(inp.q_pos.numel())
    return {"us_per_step": dt / n_seq * n_all * 1e6, "queries_timed": n_seq, "seconds": dt, "cores": threads}


def sweep_prefill(name, dev, reps=3, oracle_rows=None):
    """One-pass prefill of config `name` (C1-C3): stage times and rates."""
    cfg = CONFIGS[name]
    inp = synth.make_prefill(cfg, device=dev)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, cfg.L, cfg.L, cfg.k, cfg.h, device=dev)
    kv_slot = inp.kv_slot_table[0].long()
    run_prefill_step(cfg, inp, st, kv_slot)
    torch.cuda.synchronize()
    timer = StageTimer(["store", "indexer", "topk", "mla"])
    t0 = time.perf_counter()
    for _ in range(reps):
        run_prefill_step(cfg, inp, st, kv_slot, timer)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    stg = timer.avg_ms()
    w = prefill_work(cfg.L, cfg.k, cfg.h_i, cfg.d_i, cfg.h)
    out = {"L": cfg.L, "k": cfg.k, "indexer": f"{cfg.h_i}x{cfg.d_i}", "mla_heads": cfg.h, "ms_per_pass": wall * 1e3,
           "tokens_per_s": cfg.L / wall, "stages_ms": stg,
           "indexer_frac_fp8": w["indexer_flops"] / (stg["indexer"] * 1e-3) / 1e12 / PEAK_FP8,
           "topk_GBps": w["topk_bytes"] / (stg["topk"] * 1e-3) / 1e9,
           "mla_frac_bf16": w["mla_flops"] / (stg["mla"] * 1e-3) / 1e12 / PEAK_BF16}
    if oracle_rows:
        rows = np.linspace(0, cfg.L - 1, min(oracle_rows, cfg.L)).round().astype(np.int64)
        out["oracle"] = oracle_prefill_rate(inp, cfg, rows, cfg.L)
    del st, inp
    torch.cuda.empty_cache()
    return out


def sweep_chunked(dev, oracle_rows=64):
    """C5: one 131072-token sequence in 8192-token chunks against its growing
    prefix, FP8 latent cache: per-chunk stage times, totals and the oracle on a
    sample of rows."""
    cfg = CONFIGS["C5"]
    L, C, k = cfg.L, cfg.chunk, cfg.k
    inp = synth.make_prefill(cfg, device=dev, materialize_q=False)
    st = P.alloc_prefill(inp.n_pages, cfg.d_i, inp.n_slots, C, L, k, cfg.h, kv_fp8=True, device=dev)
    kv_slot = inp.kv_slot_table[0].long()
    chunks = []
    t_all = time.perf_counter()
    for c0 in range(0, L, C):
        c1 = c0 + C
        q = inp.q_chunk(c0, c1)
        torch.cuda.synchronize()
        timer = StageTimer(["store", "indexer", "topk", "mla"])
        t0 = time.perf_counter()
        e = timer.mark("store")
        P.store_tokens(st, inp.ik[c0:c1], inp.ik_scale[c0:c1], inp.ik_slot[c0:c1], inp.kv[c0:c1], kv_slot[c0:c1])
        e.record()
        e = timer.mark("indexer")
        dsa.indexer_scores(inp.iq[c0:c1], inp.iq_scale[c0:c1], inp.w[c0:c1], st.key_cache, st.key_scale,
                           inp.page_table, inp.q_seq[c0:c1], inp.q_pos[c0:c1], st.scores)
        e.record()
        e = timer.mark("topk")
        dsa.topk(st.scores, inp.q_pos[c0:c1], k, st.idx)
        e.record()
        e = timer.mark("mla")
        dsa.sparse_mla_prefill(q, st.kv_cache, inp.kv_slot_table, inp.q_seq[c0:c1], st.idx, SM_SCALE, st.out,
                               st.lse, kv_scale=st.kv_scale)
        e.record()
        torch.cuda.synchronize()
        chunks.append({"wall_ms": (time.perf_counter() - t0) * 1e3, **timer.avg_ms()})
        del q
    total_s = time.perf_counter() - t_all
    pairs = L * (L + 1) // 2
    sel = sum(min(k, t + 1) for t in range(L))
    idx_ms = sum(c["indexer"] for c in chunks)
    mla_ms = sum(c["mla"] for c in chunks)
    out = {"L": L, "chunk": C, "kv": "fp8_e4m3 + scale", "seconds_total": total_s, "tokens_per_s": L / total_s,
           "stages_ms_total": {s2: sum(c[s2] for c in chunks) for s2 in ("store", "indexer", "topk", "mla")},
           "last_chunk_ms": chunks[-1],
           "indexer_frac_fp8": 2.0 * cfg.h_i * cfg.d_i * pairs / (idx_ms * 1e-3) / 1e12 / PEAK_FP8,
           "mla_frac_bf16": 2.0 * cfg.h * (576 + 512) * sel / (mla_ms * 1e-3) / 1e12 / PEAK_BF16}
    if oracle_rows:
        rows = np.linspace(0, L - 1, oracle_rows).round().astype(np.int64)
        out["oracle"] = oracle_prefill_rate(inp, cfg, rows, L)
    del st, inp
    torch.cuda.empty_cache()
    return out


def sweep_configs(args, dev):
    """Every config once (C1-C3 prefill, C4 decode, C5 chunked prefill with an FP8
    latent cache), with oracle rates on row samples: one JSON object."""
    res = {}
    for name, orows in (("C1", 1024), ("C2", 128), ("C3", 128)):
        log(f"[configs] {name}")
        res[name] = sweep_prefill(name, dev, oracle_rows=orows)
        log(f"[configs] {name}: {res[name]['ms_per_pass']:.2f} ms")
    log("[configs] C4")
    dcfg, dinp, caches, newest, ds, kv_slot = setup_decode_c4(dev)
    dwall, dst = time_decode(args, dcfg, dinp, caches, newest, ds)
    gwall, gsame = time_decode_graph(args, dcfg, dinp, caches, newest, ds)
    db = decode_bytes(dinp, dcfg.k, dcfg.h)
    res["C4"] = {"batch": dcfg.decode_batch, "us_per_step": dwall * 1e6, "us_per_step_graph": gwall * 1e6,
                 "graph_matches_eager": gsame, "stages_us": {k2: v * 1e3 for k2, v in dst.items()},
                 "kernels": decode_kernels(db, dst)}
    res["C4"]["oracle"] = oracle_decode_rate(dinp, dcfg, n_seq=8)
    del caches, dinp, ds, kv_slot
    torch.cuda.empty_cache()
    log("[configs] C5")
    res["C5"] = sweep_chunked(dev)
    return res


# ---------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="time every config (C1-C5) once with oracle samples instead of the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    dsa.lib()
    if args.configs:
        print(json.dumps({"configs": sweep_configs(args, dev)}), flush=True)
        return

    # ---- prefill (headline)
    log("[bench] generating the 32K prefill inputs on the GPU")
    cfg, inp, st, kv_slot = setup_prefill_c3(dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_prefill_step(cfg, inp, st, kv_slot)
    torch.cuda.synchronize()
    log(f"[bench] prefill warmup done; timing {args.steps} steps")
    # the timed steps carry no instrumentation; the stages come from a second
    # pass of the same steps with events between the launches
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_prefill_step(cfg, inp, st, kv_slot)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    timer = StageTimer(["store", "indexer", "topk", "mla"])
    for _ in range(args.steps):
        run_prefill_step(cfg, inp, st, kv_slot, timer)
    torch.cuda.synchronize()
    stages = timer.avg_ms()
    ms_step = wall * 1e3
    tok_s = cfg.L / wall
    work = prefill_work(cfg.L, cfg.k, cfg.h_i, cfg.d_i, cfg.h)
    idx_tf = work["indexer_flops"] / (stages["indexer"] * 1e-3) / 1e12
    mla_tf = work["mla_flops"] / (stages["mla"] * 1e-3) / 1e12
    topk_gbs = work["topk_bytes"] / (stages["topk"] * 1e-3) / 1e9
    log(f"[bench] prefill {ms_step:.2f} ms/step, {tok_s:,.0f} tok/s; stages ms {stages}")
    per_kernel = {
        "indexer": {"bound": "mfma", "achieved": idx_tf, "peak": PEAK_FP8, "unit": "TFLOP/s",
                    "frac": idx_tf / PEAK_FP8, "ms": stages["indexer"]},
        "topk": {"bound": "hbm", "achieved": topk_gbs, "peak": PEAK_HBM, "unit": "GB/s",
                 "frac": topk_gbs / PEAK_HBM, "ms": stages["topk"]},
        "sparse_mla_prefill": {"bound": "mfma", "achieved": mla_tf, "peak": PEAK_BF16, "unit": "TFLOP/s",
                               "frac": mla_tf / PEAK_BF16, "ms": stages["mla"]},
        "cache_store": {"ms": stages["store"]},
    }
    dom = max(("indexer", "topk", "sparse_mla_prefill"), key=lambda n: per_kernel[n]["ms"])
    roof = {k2: v for k2, v in per_kernel[dom].items() if k2 != "ms"}
    roof.update({"kernel": dom, "traffic": recorded_traffic(dom)})

    result = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "prefill B=1 L=32768 causal k=2048; indexer 64x128 FP8 keys, page 64, shuffled "
                               "pages; sparse MLA 128 heads 576/512 bf16, page 1, shuffled slots",
                   "global_batch": 1, "seq_len": cfg.L, "topk": cfg.k},
        "stages_ms": stages,
        "kernels": per_kernel,
        "roofline": roof,
    }

    # ---- decode (second figure)
    if not args.no_decode:
        del st, inp
        torch.cuda.empty_cache()
        log("[bench] generating the 128K-context decode inputs on the GPU")
        dcfg, dinp, caches, newest, ds, kv_slot = setup_decode_c4(dev)
        dwall, dst = time_decode(args, dcfg, dinp, caches, newest, ds)
        db = decode_bytes(dinp, dcfg.k, dcfg.h)
        dk = decode_kernels(db, dst)
        result["decode"] = {"workload": "decode: 64 sequences x 1 query, context ~ U[32768, 131072] "
                                        f"(mean {float(dinp.lens.float().mean()):.0f}), k=2048, bf16 latent cache",
                            "us_per_step": dwall * 1e6, "tokens_per_s": dcfg.decode_batch / dwall,
                            "stages_us": {k2: v * 1e3 for k2, v in dst.items()}, "kernels": dk}
        log(f"[bench] decode {dwall * 1e6:.1f} us/step; stages us {result['decode']['stages_us']}")
        # the same step with the indexer and the top-k as two calls (rows split over workgroups)
        ds_u = P.alloc_decode(dcfg.decode_batch, int(dinp.lens.max()), dcfg.k, dcfg.h, fused=False, device=dev)
        uwall, ust = time_decode(args, dcfg, dinp, caches, newest, ds_u)
        result["decode"]["unfused"] = {"us_per_step": uwall * 1e6, "stages_us": {k2: v * 1e3 for k2, v in ust.items()},
                                       "kernels": decode_kernels(db, ust),
                                       "idx_equal_to_fused": bool(torch.equal(ds_u.idx, ds.idx))}
        log(f"[bench] decode, indexer and top-k as two calls: {uwall * 1e6:.1f} us/step; stages us "
            f"{result['decode']['unfused']['stages_us']}")
        del ds_u
        gwall, gsame = time_decode_graph(args, dcfg, dinp, caches, newest, ds)
        result["decode"]["us_per_step_graph"] = gwall * 1e6
        result["decode"]["graph_replay_matches_eager"] = gsame
        log(f"[bench] decode as a replayed graph {gwall * 1e6:.1f} us/step (outputs equal to eager: {gsame})")
        # multi-token-prediction shape: 2 query tokens per sequence over the same caches
        iq2, iqs2, w2, q2, pos2, seq2 = synth.decode_queries(dcfg, dinp.lens, 2, dev)
        dinp2 = dataclasses.replace(dinp, iq=iq2, iq_scale=iqs2, w=w2, q=q2, q_pos=pos2, q_seq=seq2)
        both = torch.stack([dinp.seq_start + dinp.lens - 2, dinp.seq_start + dinp.lens - 1], 1).reshape(-1).to(dev)
        newest2 = dict(ik=dinp.ik[both], ik_scale=dinp.ik_scale[both], ik_slot=dinp.ik_slot[both], kv=dinp.kv[both],
                       kv_slot=kv_slot[both])
        ds2 = P.alloc_decode(2 * dcfg.decode_batch, int(dinp.lens.max()), dcfg.k, dcfg.h, device=dev)
        dwall2, dst2 = time_decode(args, dcfg, dinp2, caches, newest2, ds2)
        db2 = decode_bytes(dinp2, dcfg.k, dcfg.h)
        dk2 = decode_kernels(db2, dst2, mla_traffic_key=None)   # 128 queries: other launch shapes
        result["decode_mtp2"] = {
            "workload": "the decode step above with 2 query tokens per sequence (positions N-2, N-1): 128 queries",
            "us_per_step": dwall2 * 1e6, "tokens_per_s": 2 * dcfg.decode_batch / dwall2,
            "stages_us": {k2: v * 1e3 for k2, v in dst2.items()}, "kernels": dk2}
        log(f"[bench] decode, 2 queries per sequence: {dwall2 * 1e6:.1f} us/step; stages us "
            f"{result['decode_mtp2']['stages_us']}")
        del ds2, dinp2, q2, iq2
        # the same step over an FP8 E4M3 latent cache (per-token scale)
        caches = fp8_kv_caches(caches, dinp, kv_slot)
        dwall8, dst8 = time_decode(args, dcfg, dinp, caches, newest, ds)
        mla8 = decode_bytes(dinp, dcfg.k, dcfg.h, kv_row_bytes=576 + 4)["mla_bytes"] / (dst8["mla"] * 1e-3) / 1e9
        result["decode_fp8_kv"] = {
            "workload": "the decode step above over an FP8 E4M3 latent cache (576 B + fp32 scale per token)",
            "us_per_step": dwall8 * 1e6, "tokens_per_s": dcfg.decode_batch / dwall8,
            "stages_us": {k2: v * 1e3 for k2, v in dst8.items()},
            "kernels": {"sparse_mla_decode": {"bound": "hbm", "achieved": mla8, "peak": PEAK_HBM, "unit": "GB/s",
                                              "us": dst8["mla"] * 1e3, "frac": mla8 / PEAK_HBM,
                                              "traffic": recorded_traffic("sparse_mla_decode_fp8")}}}
        log(f"[bench] decode, FP8 latent cache: {dwall8 * 1e6:.1f} us/step; stages us "
            f"{result['decode_fp8_kv']['stages_us']}")
        del caches, dinp, ds, kv_slot
        torch.cuda.empty_cache()
        inp = None

    if args.calib_copy:
        calib_copy(dev)
    result["measured_peaks"] = {"hbm_copy_GBps": measured_copy_bandwidth(dev),
                                "bf16_gemm_TFLOPs": measured_bf16_gemm(dev),
                                "fp8_gemm_TFLOPs": measured_fp8_gemm(dev),
                                "note": "1 GiB device-to-device copy (read + write bytes per second); torch bf16 "
                                        "matmul and FP8 E4M3 scaled matmul at 8192^3"}

    # ---- CPU baseline (the oracle on a bounded sample)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample of query rows")
        if inp is None:
            cfg, inp, st, kv_slot = setup_prefill_c3(dev)
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
