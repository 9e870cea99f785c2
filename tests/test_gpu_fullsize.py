"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the attention-projection shape (T=8192, K=5120, N=10240,
bf16 X), the MLP down-projection shape (T=8192, K=17408, N=5120, heavy-tailed
bf16 X) and the streamed accumulation (8192-token chunks at K=5120).

Where the oracle finishes in seconds it checks every output (Gram, storage,
GPTQ codes/scales/qerr at K=5120).  Where it cannot, it checks outputs it can
compute one by one (sampled Gram entries at K=17408; a block-diagonal Hessian of
the full size whose U the oracle builds block by block) or properties that hold
at any size: the projection onto the PSD cone is characterised by P >= 0,
P - H >= 0 and <P, P - H> = 0, and is at least as close to H as the PSD Gram
matrix it was stored from.
"""
import numpy as np
import pytest
import torch

import synthgen as g

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    m.lib()
    return m


def _relF(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _sym64(A):
    A = np.asarray(A, np.float64)
    return np.tril(A) + np.tril(A, -1).T


def _stored_path(gq, wl, X):
    """GPU: Gram of one chunk -> blob -> unpacked -> projected (all in HBM)."""
    K = wl.K
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_accumulate(H, X.to(DEV))
    blob = torch.empty(gq.hessian_tril_bytes(K), dtype=torch.uint8, device=DEV)
    gq.hessian_pack_tril(blob, H)
    Hs = torch.empty(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_unpack_tril(Hs, blob)
    P = Hs.clone()
    gq.psd_project(P, gq.workspace(gq.psd_project_workspace_size(K), DEV))
    torch.cuda.synchronize()
    return H, blob, Hs, P


def _kkt_certificates(P, Hs, eps):
    """Cholesky certificates (LAPACK through torch, fp64, a library check) for
    P + eps*mu*I >= 0 and (P - Hs) + eps*mu*I >= 0, plus the complementarity
    <P, P - Hs> relative to ||P|| ||P - Hs||."""
    P64 = P.to(torch.float64)
    H64 = Hs.to(torch.float64)
    H64 = torch.tril(H64) + torch.tril(H64, -1).T
    K = P.shape[0]
    mu = float(torch.diagonal(H64).mean())
    I = torch.eye(K, dtype=torch.float64, device=P.device)
    ok1 = int(torch.linalg.cholesky_ex(P64 + eps * mu * I).info) == 0
    N = P64 - H64
    ok2 = int(torch.linalg.cholesky_ex(N + eps * mu * I).info) == 0
    comp = float((P64 * N).sum() / (torch.linalg.norm(P64) * torch.linalg.norm(N)).clamp_min(1e-300))
    return ok1, ok2, comp, float(torch.linalg.norm(N) / torch.linalg.norm(H64))


# ------------------------------------------------------------------ K = 5120
@pytest.fixture(scope="module")
def attn(gq, orc):
    wl = g.WORKLOADS["attn5120"]
    X = g.x_chunk(wl)
    W = g.weights(wl)
    H, blob, Hs, P = _stored_path(gq, wl, X)
    return wl, X, W, H, blob, Hs, P


def test_attn_gram_full(gq, orc, attn):
    wl, X, W, H, blob, Hs, P = attn
    ref = orc.gram(X)
    low = np.tril_indices(wl.K)
    Hg = H.cpu().numpy()
    assert _relF(Hg[low], ref[low]) < 1e-5
    # mean(diag H) about 1, as on the dataset card's K=5120 tensor (by construction of the recipe)
    assert abs(np.diag(ref).mean() - 1.0) < 0.05


def test_attn_storage_bitexact(gq, orc, attn):
    wl, X, W, H, blob, Hs, P = attn
    ref = orc.pack_tril(H.cpu().numpy())
    assert np.array_equal(blob.cpu().numpy(), ref)
    assert np.array_equal(Hs.cpu().numpy().view(np.uint32), orc.unpack_tril(ref, wl.K).view(np.uint32))


def test_attn_projection_certificates(gq, orc, attn):
    wl, X, W, H, blob, Hs, P = attn
    Pn = P.cpu().numpy()
    assert np.array_equal(Pn, Pn.T)
    ok1, ok2, comp, change = _kkt_certificates(P, Hs, 1e-5)
    assert ok1 and ok2 and abs(comp) < 1e-3, (ok1, ok2, comp)
    # no farther from the stored matrix than the pre-storage PSD Gram (a feasible point)
    Hs64 = _sym64(Hs.cpu().numpy())
    H32 = _sym64(H.cpu().numpy())
    assert np.linalg.norm(Pn.astype(np.float64) - Hs64) <= np.linalg.norm(H32 - Hs64) * (1 + 1e-6)
    assert change < 0.00391          # below bf16's step (dataset card, "The fix")


def test_attn_projection_matches_eigendecomposition(gq, attn):
    """The projection at full size against the plain definition, computed here
    by LAPACK's symmetric eigensolver through numpy in fp64 (a library check,
    independent of the device path): eigenvalues of the stored Hessian clipped
    at zero and the matrix rebuilt.  The device result carries the rounding of
    its products (operands rounded to 48-bit integers per row) through the
    sign iteration, the unconverged eigenvalues below l_0 and the fp32 output:
    measured 2.6e-8 here, so 2e-7 is the regression bound (the acceptance bar
    is 1e-5)."""
    wl, X, W, H, blob, Hs, P = attn
    Hs64 = _sym64(Hs.cpu().numpy())
    w, V = np.linalg.eigh(Hs64)
    Pex = (V * np.maximum(w, 0.0)) @ V.T
    rel = np.linalg.norm(P.cpu().numpy().astype(np.float64) - Pex) / np.linalg.norm(Pex)
    print(f"attn5120 projection: relative Frobenius distance to the eigendecomposition {rel:.3e}")
    assert rel < 2e-7


@pytest.fixture(scope="module")
def attn_U(orc, attn):
    """The oracle's U of the projected K=5120 Hessian (computed once)."""
    wl, X, W, H, blob, Hs, P = attn
    st, U, mu = orc.gptq_U(P.cpu().numpy(), wl.damp)
    assert st == orc.OK
    return U


def test_attn_gptq_full(gq, orc, attn, attn_U):
    """All 10240 rows: codes, scales and qerr against the oracle run on the same
    projected Hessian, with the stored diagonal as importance."""
    wl, X, W, H, blob, Hs, P = attn
    N, K, G = wl.N[0], wl.K, wl.group
    imp = blob[: 4 * K].view(torch.float32)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q = gq.gptq_quantize(codes, scales, W.to(DEV), P, imp, G, wl.damp,
                         gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV))
    Wn, impn = W.numpy(), imp.cpu().numpy().copy()
    U = attn_U
    cg = orc.unpack_codes(codes.cpu().numpy(), K)
    sg = scales.cpu().numpy()
    oc, os_ = orc.gptq_sweep(Wn, U, G)
    ident = float((cg == oc).mean())
    rep = orc.gptq_replay(cg, sg, Wn, U, G)
    print(f"K=5120 code identity {ident:.6f}, replay {rep}")
    assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0
    assert ident >= 0.999
    qo = orc.qerr(oc, os_, Wn, impn)
    assert abs(q - qo) / qo < 1e-4


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_attn_gptq_variants(gq, orc, attn, attn_U, flags):
    """The variants (static groups, NF4, both) at full size: 96 sampled rows
    against the oracle's sweep and replay under the same U, static scales against
    round to nearest bit for bit, and the device's qerr against the oracle's qerr
    of the device's own codes over all 10240 rows.  Every decision must be
    admissible and at least 99.9% of them identical given the same history (the
    replay); the raw identity against the oracle's own trajectory is held to 99%
    under NF4 with dynamic scales, where each tie flip (about one per 160000
    decisions) is followed by a few hundred differing codes further along its row
    (the plain grid: under two hundred)."""
    wl, X, W, H, blob, Hs, P = attn
    N, K, G = wl.N[0], wl.K, wl.group
    imp = blob[: 4 * K].view(torch.float32)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q = gq.gptq_quantize_ex(codes, scales, W.to(DEV), P, imp, G, wl.damp, flags,
                            gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV))
    Wn, impn = W.numpy(), imp.cpu().numpy().copy()
    call = orc.unpack_codes(codes.cpu().numpy(), K, flags=flags)
    sall = scales.cpu().numpy()
    rows = np.sort(np.random.default_rng(flags).choice(N, 96, replace=False))
    rep = orc.gptq_replay(call[rows], sall[rows], Wn, attn_U, G, rows=rows, flags=flags)
    oc, os_ = orc.gptq_sweep(Wn, attn_U, G, rows=rows, flags=flags)
    ident = float((call[rows] == oc).mean())
    print(f"K=5120 flags {flags}: code identity {ident:.6f} on 96 rows, replay {rep}, qerr {q:.5f}")
    assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0
    assert rep["exact"] >= 0.999 * call[rows].size
    assert ident >= (0.999 if flags == orc.STATIC_GROUPS else 0.99)
    if flags & orc.STATIC_GROUPS:
        _, rs = orc.rtn(Wn, G, flags=flags & orc.NF4)
        assert np.array_equal(sall, rs)
    assert q == pytest.approx(orc.qerr(call, sall, Wn, impn, flags=flags), rel=1e-6)


def test_attn_gptq_act_order(gq, orc, attn):
    """Act order with static groups at full size: the device's codes, put in the
    order of decreasing diag(P), against the oracle's sweep and replay of 96
    sampled rows of the permuted problem (U of the permuted P, each column with
    its original group); scales are round to nearest's bit for bit."""
    wl, X, W, H, blob, Hs, P = attn
    N, K, G = wl.N[0], wl.K, wl.group
    flags = gq.GQ_STATIC_GROUPS | gq.GQ_ACT_ORDER
    imp = blob[: 4 * K].view(torch.float32)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q = gq.gptq_quantize_ex(codes, scales, W.to(DEV), P, imp, G, wl.damp, flags,
                            gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, flags), DEV))
    Pn, Wn, impn = P.cpu().numpy(), W.numpy(), imp.cpu().numpy().copy()
    perm = orc.act_order_perm(Pn)
    assert not np.array_equal(perm, np.arange(K))
    st, Up, _ = orc.gptq_U(_sym64(Pn)[np.ix_(perm, perm)].astype(np.float32), wl.damp)
    assert st == orc.OK
    call = orc.unpack_codes(codes.cpu().numpy(), K)
    sall = scales.cpu().numpy()
    rows = np.sort(np.random.default_rng(5).choice(N, 96, replace=False))
    Wp = np.ascontiguousarray(Wn[:, perm])
    rep = orc.gptq_replay(call[rows][:, perm], sall[rows], Wp, Up, G, rows=rows, flags=orc.STATIC_GROUPS,
                          gidx=perm // G)
    oc, _ = orc.gptq_sweep(Wp, Up, G, rows=rows, flags=orc.STATIC_GROUPS, gidx=perm // G)
    ident = float((call[rows][:, perm] == oc).mean())
    print(f"K=5120 act order: code identity {ident:.6f} on 96 rows, replay {rep}, qerr {q:.5f}")
    assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0
    assert rep["exact"] >= 0.999 * oc.size
    assert ident >= 0.99
    _, rs = orc.rtn(Wn, G)
    assert np.array_equal(sall, rs)
    assert q == pytest.approx(orc.qerr(call, sall, Wn, impn), rel=1e-6)


def test_attn_raw_stored_hessian_needs_projection(gq, orc, attn):
    """The dataset card: a stored Hessian fails Cholesky at small damping on about
    half the K=5120 tensors, and succeeds at damp 0.01 once projected.  On this
    synthetic recipe the raw stored matrix's outcome is reported, not assumed;
    the projected one must factor."""
    wl, X, W, H, blob, Hs, P = attn
    K = wl.K
    U = torch.empty(K, K, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_factor_workspace_size(K), DEV)
    gq.gptq_factor(U, P, 0.01, ws)
    try:
        gq.gptq_factor(U, Hs, 0.01, ws)
        raw = "factors"
    except gq.GQError as e:
        assert e.status == gq.GQ_ERR_NOT_PD
        raw = "NOT_PD"
    print(f"raw stored K=5120 Hessian at damp 0.01: {raw}")


# ------------------------------------------------------------------ K = 17408
@pytest.fixture(scope="module")
def mlp(gq):
    wl = g.WORKLOADS["mlpdown17408"]
    X = g.x_chunk(wl)
    H, blob, Hs, P = _stored_path(gq, wl, X)
    return wl, X, H, blob, Hs, P


@pytest.fixture(scope="module")
def mlp_w():
    return g.weights(g.WORKLOADS["mlpdown17408"])


def test_mlp_gram_sampled_entries(gq, orc, mlp):
    wl, X, H, blob, Hs, P = mlp
    K = wl.K
    rng = np.random.default_rng(0)
    I = np.concatenate([rng.integers(0, K, 200), [0, K - 1, K - 1, 5000, 17407]])
    J = np.concatenate([rng.integers(0, K, 200), [0, 0, K - 1, 4999, 128]])
    I, J = np.maximum(I, J), np.minimum(I, J)
    ref = orc.gram_entries(X, I, J)
    got = H.cpu().numpy()[I, J]
    assert _relF(got, ref) < 1e-5


def test_mlp_storage_bitexact(gq, orc, mlp):
    wl, X, H, blob, Hs, P = mlp
    ref = orc.pack_tril(H.cpu().numpy())
    assert np.array_equal(blob.cpu().numpy(), ref)
    assert np.array_equal(Hs.cpu().numpy().view(np.uint32), orc.unpack_tril(ref, wl.K).view(np.uint32))


def test_mlp_projection_certificates(gq, mlp):
    wl, X, H, blob, Hs, P = mlp
    Pc = P.cpu()
    assert torch.equal(Pc, Pc.T)
    ok1, ok2, comp, change = _kkt_certificates(P, Hs, 1e-5)
    assert ok1 and ok2 and abs(comp) < 1e-3, (ok1, ok2, comp)
    Hs64 = Hs.to(torch.float64)
    H64 = H.to(torch.float64)
    Hsym = torch.tril(H64) + torch.tril(H64, -1).T          # the GPU Gram fills the lower triangle
    assert float(torch.linalg.norm(P.to(torch.float64) - Hs64)) <= float(
        torch.linalg.norm(Hsym - Hs64)) * (1 + 1e-6)
    assert change < 0.00391


@pytest.fixture(scope="module")
def mlp_blockdiag(orc):
    """A block-diagonal K=17408 Hessian with ragged 300-column blocks (coupling
    crosses the 128-column lazy blocks) and the oracle's U, built block by block."""
    wl = g.WORKLOADS["mlpdown17408"]
    K = wl.K
    edges = list(range(0, K, 300)) + [K]
    Hd = np.zeros((K, K), np.float32)
    U = np.zeros((K, K), np.float64)
    for a, b in zip(edges[:-1], edges[1:]):
        Xb = g.normal_matrix(a + 7, g.S_X, 2 * (b - a), b - a).numpy()
        Hb = orc.gram(Xb).astype(np.float32)
        Hd[a:b, a:b] = Hb
    mu = float(np.trace(Hd.astype(np.float64)) / K)
    for a, b in zip(edges[:-1], edges[1:]):
        # the damping is in units of the whole matrix's mean diagonal
        blk = Hd[a:b, a:b].astype(np.float64) + 0.01 * mu * np.eye(b - a)
        st, Ub, _ = orc.gptq_U(blk.astype(np.float32), 0.0)
        assert st == orc.OK
        U[a:b, a:b] = Ub
    return Hd, U


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_mlp_gptq_blockdiag_hessian(gq, orc, mlp_w, mlp_blockdiag, flags):
    """Full K=17408 launch configuration (N=5120, G=128) on the block-diagonal
    Hessian, plain and with static groups, NF4 or both; the oracle sweeps sampled
    rows under its own U.  The plain sweep keeps 99.9% raw identity; the variants
    must have every decision admissible and 99.9% of them identical given the
    same history, and 99% raw identity (a tie flip on one of five 17408-wide rows
    can move a few hundred later codes)."""
    wl = g.WORKLOADS["mlpdown17408"]
    K, N, G = wl.K, wl.N[0], wl.group
    W = mlp_w
    Hd, U = mlp_blockdiag
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q = gq.gptq_quantize_ex(codes, scales, W.to(DEV), torch.from_numpy(Hd).to(DEV), None, G, 0.01, flags,
                            gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, flags), DEV))
    rows = np.array([0, 1, 777, 2500, N - 1])
    cg = orc.unpack_codes(codes.cpu().numpy()[rows], K, flags=flags)
    sg = scales.cpu().numpy()[rows]
    Wn = W.numpy()
    rep = orc.gptq_replay(cg, sg, Wn, U, G, rows=rows, flags=flags)
    oc, os_ = orc.gptq_sweep(Wn, U, G, rows=rows, flags=flags)
    ident = float((cg == oc).mean())
    print(f"K=17408 block-diagonal, flags {flags}: identity {ident:.6f}, replay {rep}")
    assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0
    assert rep["exact"] >= 0.999 * cg.size
    assert ident >= (0.999 if flags == 0 else 0.99)
    if flags & orc.STATIC_GROUPS:
        _, rs = orc.rtn(Wn[rows], G, flags=flags & orc.NF4)
        assert np.array_equal(sg, rs)
    assert 0.0 < q < 1.0


def test_mlp_gptq_diagonal_is_rtn(gq, orc, mlp_w):
    wl = g.WORKLOADS["mlpdown17408"]
    K, N, G = wl.K, wl.N[0], wl.group
    W = mlp_w
    d = np.exp(g.normal_tensor(1, g.S_S, (K,)).numpy()).astype(np.float32)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    gq.gptq_quantize(codes, scales, W.to(DEV), torch.diag(torch.from_numpy(d)).to(DEV), None, G, 0.01,
                     gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV), want_qerr=False)
    rc, rs = orc.rtn(W.numpy(), G)
    assert np.array_equal(orc.unpack_codes(codes.cpu().numpy(), K), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def test_mlp_gptq_projected_beats_rtn_on_output(gq, orc, mlp, mlp_w):
    """GPTQ with the projected K=17408 Hessian at damp 0.01 (which the dataset
    card says needs the projection) factors, and its output error ||(W - Q) X||
    on a row sample is below round-to-nearest's."""
    wl, X, H, blob, Hs, P = mlp
    K, N, G = wl.K, wl.N[0], wl.group
    W = mlp_w
    imp = blob[: 4 * K].view(torch.float32)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    q = gq.gptq_quantize(codes, scales, W.to(DEV), P, imp, G, wl.damp,
                         gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV))
    rows = np.arange(0, N, 40)
    cg = orc.unpack_codes(codes.cpu().numpy()[rows], K).astype(np.float64)
    sg = scales.cpu().numpy()[rows].astype(np.float64)
    Wr = W.numpy()[rows].astype(np.float64)
    Qg = (cg.reshape(len(rows), -1, G) * sg[:, :, None]).reshape(len(rows), K)
    rc, rs = orc.rtn(W.numpy()[rows], G)
    Qr = (rc.astype(np.float64).reshape(len(rows), -1, G) * rs[:, :, None]).reshape(len(rows), K)
    Xd = X.to(DEV).to(torch.float64)
    eg = float(torch.linalg.norm(torch.from_numpy(Wr - Qg).to(DEV) @ Xd.T))
    er = float(torch.linalg.norm(torch.from_numpy(Wr - Qr).to(DEV) @ Xd.T))
    print(f"K=17408 qerr {q:.5f}; output error GPTQ/RTN = {eg / er:.4f}")
    assert eg < er


# ------------------------------------------------------------------ streaming
def test_stream_chunks_full_width(gq, orc):
    """8 chunks of 8192 tokens at K=5120 (the streamed recipe), accumulated in
    two halves with a host round trip of H in between: bitwise equal to the
    uninterrupted run, and equal to the oracle's sum on sampled entries."""
    wl = g.WORKLOADS["stream5120"]
    small = g.Workload("stream5120", wl.T, wl.K, wl.N, wl.group, wl.damp, "bf16", True, 8, wl.seed)
    K = wl.K
    chunks = [g.x_chunk(small, c) for c in range(small.chunks)]
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    for X in chunks:
        gq.hessian_accumulate(H, X.to(DEV))
    H2 = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    for X in chunks[:4]:
        gq.hessian_accumulate(H2, X.to(DEV))
    H3 = H2.cpu().to(DEV)
    for X in chunks[4:]:
        gq.hessian_accumulate(H3, X.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(H.cpu(), H3.cpu())
    rng = np.random.default_rng(1)
    I = rng.integers(0, K, 64)
    J = rng.integers(0, K, 64)
    I, J = np.maximum(I, J), np.minimum(I, J)
    ref = sum(orc.gram_entries(X, I, J) for X in chunks)
    assert _relF(H.cpu().numpy()[I, J], ref) < 1e-5


def test_stream_tensors_share_one_factor(gq, orc, attn, attn_U):
    """The four weight tensors of the streamed recipe (N = 5120, 10240, 1024 and
    1024 rows at K=5120) share one Hessian: gptq_factor runs once and gptq_sweep
    once per tensor under that U.  On 96 sampled rows of each tensor, the
    oracle's replay under its own U of the same projected Hessian finds every
    decision admissible and 99.9% of them identical given the same history; raw
    identity with the oracle's own sweep is held to 99% (a single legitimate tie
    flip moves a few hundred later codes of its 5120-wide row).  The last
    tensor's codes, scales and qerr equal gptq_quantize's bytes."""
    wl, X, W0, H, blob, Hs, P = attn
    sw = g.WORKLOADS["stream5120"]
    K, G = sw.K, sw.group
    U = torch.empty(K, K, dtype=torch.float32, device=DEV)
    gq.gptq_factor(U, P, sw.damp, gq.workspace(gq.gptq_factor_workspace_size(K), DEV))
    imp = blob[: 4 * K].view(torch.float32)
    impn = imp.cpu().numpy().copy()
    for t, N in enumerate(sw.N):
        W = g.weights(sw, t)
        Wd = W.to(DEV)
        codes = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
        scales = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
        ws = gq.workspace(gq.gptq_sweep_workspace_size(N, K, G), DEV)
        q = gq.gptq_sweep(codes, scales, Wd, U, imp, G, ws)
        Wn = W.numpy()
        rows = np.sort(np.random.default_rng(t).choice(N, 96, replace=False))
        cg = orc.unpack_codes(codes.cpu().numpy()[rows], K)
        sg = scales.cpu().numpy()[rows]
        rep = orc.gptq_replay(cg, sg, Wn, attn_U, G, rows=rows)
        oc, _ = orc.gptq_sweep(Wn, attn_U, G, rows=rows)
        ident = float((cg == oc).mean())
        print(f"stream tensor {t} (N={N}): identity {ident:.6f}, replay {rep}, qerr {q:.5f}")
        assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0
        assert rep["exact"] >= 0.999 * cg.size and ident >= 0.99
        assert q == pytest.approx(orc.qerr(orc.unpack_codes(codes.cpu().numpy(), K), scales.cpu().numpy(), Wn, impn),
                                  rel=1e-6)
    c2 = torch.empty_like(codes)
    s2 = torch.empty_like(scales)
    q2 = gq.gptq_quantize(c2, s2, Wd, P, imp, G, sw.damp,
                          gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV))
    assert torch.equal(c2, codes) and torch.equal(s2, scales) and q2 == q
