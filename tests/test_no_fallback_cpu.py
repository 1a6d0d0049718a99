"""The product path has no CPU fallback: without the built library, or with
host tensors, its calls raise (runs without a GPU)."""
import pytest
import torch

from long_context_sparse_hisa_amd import hisa


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(hisa, "_lib", None)
    monkeypatch.setattr(hisa, "LIB_PATH", str(tmp_path / "libhisa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hisa.lib()
    with pytest.raises(RuntimeError, match="not built"):
        hisa.abi_version()


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="GPU tensor"):
        hisa._dev(torch.zeros(4, dtype=torch.int32), "out_idx")
    assert hisa._dev(None, "out_scores") is None
