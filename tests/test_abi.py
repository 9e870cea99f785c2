"""CPU checks of the C ABI library: it loads without a GPU and exports every
symbol include/gq.h declares (no compute calls: there is no GPU here)."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_accumulate_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "gq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "while", "for", "sizeof"})


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(gq.EXPORTS)


@pytest.mark.skipif(not os.path.exists(gq.LIB_PATH), reason="libgq.so not built")
def test_library_loads_and_exports_every_symbol():
    L = ctypes.CDLL(gq.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name
    assert gq.abi_version() == 1


@pytest.mark.skipif(not os.path.exists(gq.LIB_PATH), reason="libgq.so not built")
def test_size_queries_are_host_only():
    # Bf16TrilDiagF32 size: K*4 + K*(K-1)/2*2 (hipfire-calib-data, "Hessian storage")
    for K, n in [(128, 16768), (1024, 1051648), (5120, 26229760), (17408, 303090688)]:
        assert gq.hessian_tril_bytes(K) == n
    assert gq.hessian_tril_bytes(0) == 0
    assert gq.psd_project_workspace_size(1024) >= 4 * 1024 * 1024 * 8
    assert gq.gptq_quantize_workspace_size(64, 128, 32) > gq.gptq_sweep_workspace_size(64, 128, 32)
    # every round-to-nearest workspace fits the fixed scratch of rtn_quantize_noalloc
    for N, K, G in [(1, 2, 1), (10240, 5120, 128), (5120, 17408, 128), (1 << 20, 8192, 1), (7, 130, 2)]:
        assert gq.rtn_quantize_workspace_size(N, K, G) <= gq.NOALLOC_SCRATCH_BYTES


@pytest.mark.skipif(not os.path.exists(gq.LIB_PATH), reason="libgq.so not built")
def test_product_kind_switch_is_host_only():
    # The workspace covers both kinds of product, so its size does not move.
    n = gq.psd_project_workspace_size(5120)
    gq.gq_set_psd_products(gq.GQ_PSD_F64)
    assert gq.psd_project_workspace_size(5120) == n
    gq.gq_set_psd_products(gq.GQ_PSD_AUTO)
    with pytest.raises(gq.GQError):
        gq.gq_set_psd_products(7)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gq, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        gq.lib()


@pytest.mark.skipif(not os.path.exists(gq.LIB_PATH), reason="libgq.so not built")
def test_nf4_table_is_the_oracles(orc):
    """The library's NF4 levels (literals in its source) are the oracle's (built
    from scipy's normal quantile function), bit for bit; host-only call."""
    import numpy as np
    lib_levels = gq.nf4_levels().numpy()
    assert np.array_equal(lib_levels.view(np.uint32), orc.nf4_levels().view(np.uint32))
