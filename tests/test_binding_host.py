"""The Python binding on the host (no GPU): it marshals device tensors only
and has no CPU path, so host tensors, wrong dtypes and non-contiguous views
are refused before anything reaches the library, and a missing library is an
ImportError."""
import pytest
import torch

import long_context_sparse_fp8_amd as dsa
import long_context_sparse_fp8_amd._binding as B


def test_host_tensors_are_refused():
    s = torch.zeros(4, 100)
    pos = torch.zeros(4, dtype=torch.int32)
    idx = torch.zeros(4, 16, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.topk(s, pos, 16, idx)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.kv_cache_store(torch.zeros(2, 576, dtype=torch.bfloat16), torch.zeros(2, dtype=torch.int64),
                           torch.zeros(8, 576, dtype=torch.bfloat16))


def test_dtypes_and_layout_are_checked():
    with pytest.raises(TypeError, match="expected torch.float32"):
        B._ptr(torch.zeros(3, dtype=torch.float64), torch.float32, "scores")
    with pytest.raises(TypeError, match="torch.Tensor"):
        B._ptr([1, 2, 3], None, "scores")
    assert B._ptr(None) is None


def test_fp8_cache_needs_its_scales():
    n, h = 2, 128
    q = torch.zeros(n, h, 576, dtype=torch.bfloat16)
    cache = torch.zeros(8, 576, dtype=torch.uint8)
    with pytest.raises(ValueError, match="kv_scale"):
        dsa.sparse_mla_prefill(q, cache, torch.zeros(1, 8, dtype=torch.int32), torch.zeros(n, dtype=torch.int32),
                               torch.zeros(n, 16, dtype=torch.int32), 1 / 24,
                               torch.zeros(n, h, 512, dtype=torch.bfloat16))


def test_missing_library_is_an_import_error(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libdsa.so"))
    with pytest.raises(ImportError, match="missing"):
        B.lib()
