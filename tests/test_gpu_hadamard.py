"""GPU parity of the block Walsh-Hadamard rotation (hadamard_rotate_rows,
hadamard_rotate_hessian) against the oracle's dense fp64 rotation, through the C
ABI.  The device runs log2(b) fp32 butterfly stages, so the bar is 1e-5 relative
Frobenius (the Hessian bar), with every entry checked.  Shapes: blocks of 1 to
4096 (the Hessian's below 16 take the in-place kernel and a copy back), a row
stride above K, signs or none, the bench workload's W (10240 x 5120,
b = 1024) on sampled rows and its K = 5120 Hessian; plus the output invariance
and the rotated path through GPTQ."""
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


def _relF(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _signs(K, seed):
    return np.random.default_rng(seed).choice([-1.0, 1.0], K).astype(np.float32)


@pytest.mark.parametrize("rows,K,b,extra,signed", [
    (37, 256, 256, 0, True), (64, 1024, 1024, 0, False), (10, 96, 32, 4, True), (5, 4096, 4096, 0, True),
    (7, 12, 4, 0, False), (3, 6, 2, 0, True), (2, 5, 1, 3, True), (300, 2048, 64, 0, True)])
def test_rotate_rows(gq, orc, rows, K, b, extra, signed):
    rng = np.random.default_rng(rows * K + b)
    A = rng.standard_normal((rows, K + extra)).astype(np.float32)
    s = _signs(K, b) if signed else None
    Ad = torch.from_numpy(A).to(DEV)
    gq.hadamard_rotate_rows(Ad[:, :K], b, torch.from_numpy(s).to(DEV) if signed else None)
    out = Ad.cpu().numpy()
    ref = orc.hadamard_rotate_rows(A[:, :K], b, s)
    assert _relF(out[:, :K], ref) < 1e-5
    assert np.abs(out[:, :K] - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-30
    assert np.array_equal(out[:, K:], A[:, K:])             # the columns past K are not touched


@pytest.mark.parametrize("K,b", [(256, 128), (1024, 1024), (96, 32), (48, 8), (20, 4), (10, 1)])
def test_rotate_hessian(gq, orc, K, b):
    rng = np.random.default_rng(K)
    X = rng.standard_normal((3 * K, K)).astype(np.float32)
    H = orc.gram(X).astype(np.float32)
    H = np.tril(H) + np.tril(H, -1).T
    s = _signs(K, 3)
    Hd = torch.from_numpy(H).to(DEV)
    ws = torch.empty(gq.hadamard_rotate_hessian_workspace_size(K), dtype=torch.uint8, device=DEV)
    gq.hadamard_rotate_hessian(Hd, b, ws, torch.from_numpy(s).to(DEV))
    out = Hd.cpu().numpy()
    ref = orc.hadamard_rotate_hessian(H, b, s)
    assert _relF(out, ref) < 1e-5
    assert _relF(out, out.T) < 1e-6                        # symmetric to rounding


def test_full_size_weights_and_hessian(gq, orc):
    wl = g.WORKLOADS["attn5120"]
    K, N, b = wl.K, wl.N[0], 1024
    W = g.weights(wl).numpy()
    s = _signs(K, 11)
    Wd = torch.from_numpy(W).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    gq.hadamard_rotate_rows(Wd, b, sd)
    rows = np.random.default_rng(0).choice(N, 64, replace=False)
    R = orc.hadamard_rotation(K, b, s)
    ref = (W[rows].astype(np.float64) @ R.T)
    assert _relF(Wd.cpu().numpy()[rows], ref) < 1e-5
    # the Hessian of the workload's activations, rotated, against R H R^T in fp64
    X = g.x_chunk(wl, device=DEV)
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_accumulate(H, X)
    Hs = torch.tril(H) + torch.tril(H, -1).T
    H64 = Hs.cpu().numpy().astype(np.float64)
    ws = torch.empty(gq.hadamard_rotate_hessian_workspace_size(K), dtype=torch.uint8, device=DEV)
    gq.hadamard_rotate_hessian(Hs, b, ws, sd)
    assert _relF(Hs.cpu().numpy(), R @ H64 @ R.T) < 1e-5


def test_outputs_unchanged_and_rotated_gptq(gq, orc):
    """W' X'^T = W X^T on the device, and GPTQ on the rotated pair is GPTQ on its
    inputs: the device's codes on (W R^T, R H R^T) match the oracle's on the same
    rotated inputs (the plain GPTQ parity, one step later in the path)."""
    wl = g.WORKLOADS["stored1024"]
    K, N, b = wl.K, wl.N[0], 256
    W = g.weights(wl).numpy()
    X = g.x_chunk(wl).numpy()
    s = _signs(K, 7)
    sd = torch.from_numpy(s).to(DEV)
    Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
    Y = (Wd.double() @ Xd.double().T)
    gq.hadamard_rotate_rows(Wd, b, sd)
    gq.hadamard_rotate_rows(Xd, b, sd)
    Yr = (Wd.double() @ Xd.double().T)
    assert (torch.linalg.norm(Yr - Y) / torch.linalg.norm(Y)).item() < 1e-5
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_accumulate(H, Xd)
    Hs = (torch.tril(H) + torch.tril(H, -1).T).cpu().numpy()
    Wn = Wd.cpu().numpy()
    # the plain GPTQ parity check (codes, and scales under the oracle's replay of
    # the device's decisions) on the rotated inputs; qerr parity is tested on its own
    from test_gpu_parity import _check_gptq, _gpu_gptq
    codes, scales, _ = _gpu_gptq(gq, Wn, Hs, wl.group, wl.damp, want_qerr=False)
    _check_gptq(orc, Wn, Hs, wl.group, codes, scales, None, damp=wl.damp)
