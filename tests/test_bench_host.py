"""Host-side checks of the benchmark script (no GPU needed): the one-GPU
guard, the algorithmic work counts that the roofline fractions divide by,
and the rule that recorded HBM traffic is reported only for unchanged
kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_work_closed_forms():
    L, k = 32768, 2048
    w = bench.prefill_work(L, k, 64, 128, 128)
    assert w["pairs"] == L * (L + 1) // 2
    # rows 0..k-1 keep every predecessor, later rows exactly k
    assert w["selected_pairs"] == k * (k + 1) // 2 + (L - k) * k
    assert w["indexer_flops"] == 2.0 * 64 * 128 * L * (L + 1) / 2
    assert w["mla_flops"] == 2.0 * 128 * (576 + 512) * w["selected_pairs"]
    assert abs(w["indexer_flops"] - 8.80e12) / 8.80e12 < 5e-3
    assert abs(w["mla_flops"] - 1.81e13) / 1.81e13 < 5e-3
    # rows longer than k are read whole; every row writes k indices
    assert w["topk_bytes"] == 4.0 * sum(range(k + 1, L + 1)) + 4.0 * L * k
    tiny = bench.prefill_work(4, 8, 16, 64, 8)
    assert tiny["selected_pairs"] == tiny["pairs"] == 10 and tiny["topk_bytes"] == 4.0 * 4 * 8


def test_recorded_traffic_needs_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "kern.hip"
    src.write_text("kernel source\n")
    import hashlib
    digest = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    rec = tmp_path / "traffic.txt"
    rel = os.path.relpath(str(src), ROOT)
    rec.write_text(f"# header\nkernel=k1 name=x grid=1 fetch_bytes=10 write_bytes=5 traffic_bytes=15 "
                   f"sources={rel} sha256={digest}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic("k1") == 15.0
    assert bench.recorded_traffic("k2") is None
    src.write_text("kernel source, changed\n")
    assert bench.recorded_traffic("k1") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic("k1") is None



def test_decode_kernels_fused_and_split_stages(tmp_path, monkeypatch):
    """The decode roofline lines: a fused indexer -> top-k stage carries the bytes of
    both stages and the recorded traffic of its three launches (null while any is
    missing); the two-call form reports the stages apart; the 128-query step gets
    no traffic from the 64-query launches."""
    import hashlib
    src = tmp_path / "kern.hip"
    src.write_text("kernel source\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    rel = os.path.relpath(str(src), ROOT)
    line = lambda name, t: (f"kernel={name} name=x grid=1 fetch_bytes={t} write_bytes=0 traffic_bytes={t} "
                            f"sources={rel} sha256={digest}\n")
    rec = tmp_path / "traffic.txt"
    rec.write_text(line("indexer_decode", 700) + line("topk_fused_part", 20) + line("topk_fused_merge", 3) +
                   line("sparse_mla_decode", 190))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    db = {"indexer_bytes": 8.0e8, "topk_bytes": 2.0e7, "mla_bytes": 1.6e8}
    fused = bench.decode_kernels(db, {"store": 0.01, "indexer_topk": 0.2, "mla": 0.08})
    assert set(fused) == {"indexer_topk", "sparse_mla_decode"}
    assert fused["indexer_topk"]["achieved"] == (8.0e8 + 2.0e7) / 0.2e-3 / 1e9
    assert fused["indexer_topk"]["traffic"] == 723.0
    assert fused["sparse_mla_decode"]["traffic"] == 190.0
    assert abs(fused["sparse_mla_decode"]["frac"] - 1.6e8 / 0.08e-3 / 1e9 / bench.PEAK_HBM) < 1e-12
    split = bench.decode_kernels(db, {"store": 0.01, "indexer": 0.15, "topk": 0.04, "mla": 0.08})
    assert set(split) == {"indexer", "topk", "sparse_mla_decode"}
    assert split["topk"]["achieved"] == 2.0e7 / 0.04e-3 / 1e9
    mtp = bench.decode_kernels(db, {"store": 0.01, "indexer_topk": 0.2, "mla": 0.1}, mla_traffic_key=None)
    assert mtp["sparse_mla_decode"]["traffic"] is None
    rec.write_text(line("indexer_decode", 700) + line("sparse_mla_decode", 190))
    assert bench.decode_kernels(db, {"indexer_topk": 0.2, "mla": 0.08})["indexer_topk"]["traffic"] is None
