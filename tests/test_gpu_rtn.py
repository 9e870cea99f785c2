"""GPU parity of rtn_quantize -- round to nearest on the GPTQ int4 grid, with no
error feedback -- against the oracle's RTN, through the C ABI.

Both sides take every decision in fp32 (scale = absmax/7 by an IEEE division,
code = rint(w / scale) by an IEEE division, ties to even), so codes and scales
are compared bit for bit; qerr is a ratio of fp64 sums on both sides, summed in
different orders, so it is compared to 1e-9 relative.  Shapes cover the vector
kernel (K a multiple of 8, groups of 1 to 128 columns) and the generic one (K not
a multiple of 8, or W not 16-byte aligned), a ragged row count, an all-zero
group and exact ties.  At the bench workload's full size (10240 x 5120, groups
of 128) the codes are checked against the oracle too, and qerr of uniform
weights against the closed form behind the wiki's uniform-weight check.
"""
import math

import numpy as np
import pytest
import torch

import synthgen as g

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _gpu_rtn(gq, W, G, imp=None, want_qerr=True, offset=0):
    """Codes (N x K/2 bytes), scales (N x K/G) and qerr of the device RTN; with
    offset > 0, W is a view starting `offset` floats into its allocation."""
    N, K = W.shape
    if offset:
        buf = torch.zeros(N * K + offset, dtype=torch.float32, device=DEV)
        Wd = buf[offset:].view(N, K)
        Wd.copy_(torch.from_numpy(W))
    else:
        Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    codes = torch.empty(N * (K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty(N * (K // G), dtype=torch.float32, device=DEV)
    ws = torch.empty(gq.rtn_quantize_workspace_size(N, K, G), dtype=torch.uint8, device=DEV)
    impd = torch.from_numpy(imp).to(DEV) if imp is not None else None
    q = gq.rtn_quantize(codes, scales, Wd, impd, G, ws, want_qerr)
    torch.cuda.synchronize()
    return codes.cpu().numpy().reshape(N, K // 2), scales.cpu().numpy().reshape(N, K // G), q


def _weights(N, K, G, seed):
    """Normal weights with an all-zero group, a row of exact ties (absmax 7, so
    scale 1, and values k + 1/2) and a few exact zeros."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)).astype(np.float32)
    W[rng.integers(0, N, 5), rng.integers(0, K, 5)] = 0.0
    W[0, :G] = 0.0
    if N > 1 and G >= 2:
        ties = np.array([7.0, 2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -6.5], np.float32)
        W[1, :G] = np.resize(ties, G)
    return W


SHAPES = [
    # (N, K, G, offset)
    (37, 256, 32, 0),
    (64, 1024, 128, 0),
    (5, 2048, 8, 0),
    (9, 64, 4, 0),
    (9, 64, 2, 0),
    (9, 64, 1, 0),
    (3, 6, 2, 0),        # K % 8 != 0: generic kernel
    (3, 12, 4, 0),
    (4, 10, 1, 0),
    (7, 256, 32, 1),     # W not 16-byte aligned: generic kernel
    (1, 2, 1, 0),        # smallest shape
    (1, 8, 8, 0),
]


@pytest.mark.parametrize("N,K,G,offset", SHAPES)
def test_rtn_bitexact(gq, orc, N, K, G, offset):
    W = _weights(N, K, G, seed=N * 1000 + K + G)
    codes, scales, q = _gpu_rtn(gq, W, G, offset=offset)
    rc, rs = orc.rtn(W, G)
    assert np.array_equal(orc.unpack_codes(codes, K), rc)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, orc.pack_codes(rc))
    assert q == pytest.approx(orc.qerr(rc, rs, W), rel=1e-9, abs=1e-15)


def test_rtn_ties_and_zero_group(gq, orc):
    W = _weights(4, 64, 8, seed=3)
    codes, scales, _ = _gpu_rtn(gq, W, 8)
    c = orc.unpack_codes(codes, 64)
    assert scales[0, 0] == 0.0 and (c[0, :8] == 0).all()            # all-zero group
    assert scales[1, 0] == 1.0                                      # absmax 7
    assert c[1, :8].tolist() == [7, 2, -2, 0, 0, 2, 4, -6]           # ties to even


def test_rtn_qerr_request_and_importance(gq, orc):
    W = g.uniform_weights(9, 128, 256).numpy()
    a = _gpu_rtn(gq, W, 64)
    b = _gpu_rtn(gq, W, 64, want_qerr=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and b[2] is None
    ones = _gpu_rtn(gq, W, 64, imp=np.ones(256, np.float32))
    assert ones[2] == pytest.approx(a[2], rel=1e-12)
    imp = np.exp(np.random.default_rng(0).standard_normal(256)).astype(np.float32)
    qi = _gpu_rtn(gq, W, 64, imp=imp)
    assert np.array_equal(qi[0], a[0])                               # the pack does not move
    assert qi[2] != a[2]                                              # an imatrix moves qerr
    rc, rs = orc.rtn(W, 64)
    assert qi[2] == pytest.approx(orc.qerr(rc, rs, W, imp), rel=1e-9)
    assert _gpu_rtn(gq, W, 64, imp=imp)[2] == qi[2]                   # deterministic


def test_rtn_full_size_uniform(gq, orc):
    """Bench-sized uniform weights (10240 x 5120, groups of 128): codes and scales
    as the oracle's, and qerr at the closed form sqrt((G-1)/(G+2))/14 (the group
    maximum is exact, the other errors uniform over one step of absmax/7), the
    wiki's 0.0714 for large groups."""
    wl = g.WORKLOADS["attn5120"]
    N, K, G = wl.N[0], wl.K, wl.group
    W = g.uniform_weights(11, N, K).numpy()
    codes, scales, q = _gpu_rtn(gq, W, G)
    rc, rs = orc.rtn(W, G)
    assert np.array_equal(codes, orc.pack_codes(rc))
    assert np.array_equal(scales, rs)
    assert q == pytest.approx(math.sqrt((G - 1) / (G + 2)) / 14.0, rel=2e-3)
    assert q == pytest.approx(orc.qerr(rc, rs, W), rel=1e-9)


def test_rtn_full_size_bench_weights(gq, orc):
    """The bench workload's own synthetic weights: pack bit-exact against the oracle."""
    wl = g.WORKLOADS["attn5120"]
    W = g.weights(wl).numpy()
    codes, scales, q = _gpu_rtn(gq, W, wl.group)
    rc, rs = orc.rtn(W, wl.group)
    assert np.array_equal(codes, orc.pack_codes(rc))
    assert np.array_equal(scales, rs)
    assert q == pytest.approx(orc.qerr(rc, rs, W), rel=1e-9)


def test_rtn_errors(gq):
    W = np.ones((4, 64), np.float32)
    W[2, 5] = np.nan
    with pytest.raises(gq.GQError) as e:
        _gpu_rtn(gq, W, 32)
    assert e.value.status == gq.GQ_ERR_NONFINITE
    imp = np.ones(64, np.float32)
    imp[3] = np.inf
    with pytest.raises(gq.GQError) as e:
        _gpu_rtn(gq, np.ones((4, 64), np.float32), 32, imp=imp)
    assert e.value.status == gq.GQ_ERR_NONFINITE
    for G in (3, 256, 64):                        # not a power of two, above 128, not dividing K
        with pytest.raises(gq.GQError) as e:
            Wd = torch.ones(4, 96, device=DEV)
            codes = torch.empty(4 * 48, dtype=torch.uint8, device=DEV)
            scales = torch.empty(4 * 96, dtype=torch.float32, device=DEV)
            ws = torch.empty(gq.rtn_quantize_workspace_size(4, 96, 32), dtype=torch.uint8, device=DEV)
            gq.rtn_quantize(codes, scales, Wd, None, G, ws)
        assert e.value.status == gq.GQ_ERR_INVALID_ARG
    with pytest.raises(gq.GQError) as e:
        Wd = torch.ones(4, 64, device=DEV)
        codes = torch.empty(4 * 32, dtype=torch.uint8, device=DEV)
        scales = torch.empty(4 * 2, dtype=torch.float32, device=DEV)
        gq.rtn_quantize(codes, scales, Wd, None, 32, torch.empty(8, dtype=torch.uint8, device=DEV))
    assert e.value.status == gq.GQ_ERR_INVALID_ARG
