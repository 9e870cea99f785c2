"""GPU parity: every HIP stage against the CPU oracle on the same seeded inputs,
through the C ABI (via the thin binding), at sizes the oracle finishes in
seconds, spanning several tiles and a ragged tail.

Bars (from the stated parity standards): tril packing bit-exact; Hessians
(Gram and PSD-projected) within 1e-5 relative Frobenius; int4 codes identical on
>= 99.9% with every difference a tie flip under the oracle's replay; scales
within 1e-5 relative; qerr within 1e-4 relative.
"""
import numpy as np
import pytest
import torch

import synthgen as g

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import post_weight_quantization_accumulate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


DEV = "cuda:0"


def _relF(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _sym(A):
    A = np.asarray(A, np.float64)
    return np.tril(A) + np.tril(A, -1).T


def _gpu_gram(gq, X):
    Xd = X.to(DEV)
    K = X.shape[1]
    H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    gq.hessian_accumulate(H, Xd)
    torch.cuda.synchronize()
    return H.cpu().numpy()


# ------------------------------------------------------------------ tril storage
@pytest.mark.parametrize("K", [1, 2, 77, 128, 300, 1024])
def test_tril_pack_unpack_bitexact(gq, orc, K):
    rng = np.random.default_rng(K)
    H = rng.standard_normal((K, K)).astype(np.float32)
    bits = H.view(np.uint32)
    # special patterns: denormals, signed zero, infinities, NaN payloads, truncation edges
    specials = [0x00012345, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0x3F80C000, 0xBFFFFFFF,
                0x3F80FFFF]
    flat = bits.reshape(-1)
    flat[: min(len(specials), flat.size)] = specials[: min(len(specials), flat.size)]
    Ht = torch.from_numpy(H).to(DEV)
    blob = torch.zeros(gq.hessian_tril_bytes(K), dtype=torch.uint8, device=DEV)
    gq.hessian_pack_tril(blob, Ht)
    ref = orc.pack_tril(H)
    assert np.array_equal(blob.cpu().numpy(), ref)
    Hu = torch.full((K, K), 7.0, dtype=torch.float32, device=DEV)
    gq.hessian_unpack_tril(Hu, torch.from_numpy(ref).to(DEV))
    assert np.array_equal(Hu.cpu().numpy().view(np.uint32), orc.unpack_tril(ref, K).view(np.uint32))


# ------------------------------------------------------------------ Gram
@pytest.mark.parametrize("T,K", [(512, 128), (100, 200), (4096, 1024), (33, 260)])
def test_gram_f32_parity(gq, orc, T, K):
    X = g.normal_matrix(T + K, g.S_X, T, K)
    H = _gpu_gram(gq, X)
    ref = orc.gram(X)
    low = np.tril_indices(K)
    assert _relF(H[low], ref[low]) < 1e-5
    assert np.all(np.triu(H, 1) == 0)          # the strict upper triangle is not touched


@pytest.mark.parametrize("T,K", [(1000, 300), (8192, 1024), (37, 136), (4096, 520), (1, 8), (130, 2056),
                                 (200, 264)])
def test_gram_bf16_parity(gq, orc, T, K):
    wl = g.Workload("attn5120", T, K, [8], 128, 0.01, "bf16", True, 1, 2)
    X = g.x_chunk(wl)
    assert X.dtype == torch.bfloat16
    H = _gpu_gram(gq, X)
    ref = orc.gram(X)
    low = np.tril_indices(K)
    assert _relF(H[low], ref[low]) < 1e-5
    assert np.all(np.triu(H, 1) == 0)


def test_gram_chunks_add_and_resume_bitwise(gq, orc):
    """Streaming: chunk sums add (AtomicChat GGUF page, 'The importance matrix');
    saving H mid-stream and resuming reproduces the uninterrupted run bitwise."""
    wl = g.Workload("stream5120", 1024, 384, [8], 128, 0.01, "bf16", True, 6, 4)
    chunks = [g.x_chunk(wl, c).to(DEV) for c in range(wl.chunks)]
    H = torch.zeros(384, 384, dtype=torch.float32, device=DEV)
    for X in chunks:
        gq.hessian_accumulate(H, X)
    H2 = torch.zeros_like(H)
    for X in chunks[:3]:
        gq.hessian_accumulate(H2, X)
    saved = H2.cpu().clone()
    H3 = saved.to(DEV)
    for X in chunks[3:]:
        gq.hessian_accumulate(H3, X)
    torch.cuda.synchronize()
    assert torch.equal(H.cpu(), H3.cpu())
    ref = np.zeros((384, 384))
    for X in chunks:
        orc.gram(X.cpu(), ref)
    low = np.tril_indices(384)
    assert _relF(H.cpu().numpy()[low], ref[low]) < 1e-5


@pytest.mark.parametrize("K", [520, 256, 300])
def test_gram_chunks_call(gq, orc, K):
    """hessian_accumulate_chunks: several chunks of ragged token counts (one
    empty, one of a single token) in one call, with and without a workspace
    (workgroups sharing tiles, partial tiles added in a fixed order), against
    the oracle's sum of the chunks' Gram matrices; repeated calls are bitwise
    equal, and the result matches the chunk-by-chunk calls to fp32 rounding.
    K = 300 (not a multiple of 8) takes the chunk-by-chunk route inside."""
    Ts = [100, 37, 0, 512, 1, 64, 300, 33, 250]
    wl = g.Workload("stream5120", 512, K, [8], 128, 0.01, "bf16", True, len(Ts), 4)
    chunks = [g.x_chunk(wl, c, device=DEV, tokens=max(T, 1))[:T].contiguous() for c, T in enumerate(Ts)]
    ref = np.zeros((K, K))
    for X in chunks:
        if X.shape[0]:
            orc.gram(X.cpu(), ref)
    low = np.tril_indices(K)
    ws = gq.workspace(max(gq.hessian_accumulate_chunks_workspace_size(K, len(chunks)), 1), DEV)
    outs = []
    for w in (ws, None, ws):
        H = torch.zeros(K, K, dtype=torch.float32, device=DEV)
        gq.hessian_accumulate_chunks(H, chunks, w)
        torch.cuda.synchronize()
        Hn = H.cpu().numpy()
        assert _relF(Hn[low], ref[low]) < 1e-5
        assert np.all(np.triu(Hn, 1) == 0)
        outs.append(Hn)
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    H1 = torch.zeros(K, K, dtype=torch.float32, device=DEV)
    for X in chunks:
        gq.hessian_accumulate(H1, X)
    torch.cuda.synchronize()
    assert _relF(outs[0][low], H1.cpu().numpy()[low]) < 1e-6
    # into a non-zero H: the chunks' sum is added
    H = H1.clone()
    gq.hessian_accumulate_chunks(H, chunks, ws)
    torch.cuda.synchronize()
    assert _relF(H.cpu().numpy()[low], 2 * ref[low]) < 1e-5


def test_gram_is_deterministic(gq):
    X = g.normal_matrix(3, g.S_X, 2048, 512).to(torch.bfloat16)
    a = _gpu_gram(gq, X)
    for _ in range(5):
        assert np.array_equal(a.view(np.uint32), _gpu_gram(gq, X).view(np.uint32))


# ------------------------------------------------------------------ PSD projection
def _gpu_psd(gq, H):
    K = H.shape[0]
    Ht = torch.from_numpy(np.ascontiguousarray(H, np.float32)).to(DEV)
    ws = gq.workspace(gq.psd_project_workspace_size(K), DEV)
    gq.psd_project(Ht, ws)
    return Ht.cpu().numpy()


@pytest.mark.parametrize("K", [5, 130, 300])
def test_psd_random_indefinite(gq, orc, K):
    rng = np.random.default_rng(K)
    A = rng.standard_normal((K, K))
    H = ((A + A.T) / 2).astype(np.float32)
    P = _gpu_psd(gq, H)
    P_ref, P64 = orc.psd_project(H, 1, return_f64=True)
    assert np.array_equal(P, P.T)
    assert _relF(P, P64) < 1e-5


@pytest.mark.parametrize("kind", ["emulated", "f64"])
@pytest.mark.parametrize("K", [4100, 4112])
def test_psd_known_spectrum_ragged(gq, K, kind):
    """K=4100 and 4112: 33 tile rows of 128 (the last one 4 or 16 wide).
    Emulated products: the split forms are padded to 4352 = 17 tiles of 256,
    the last one mostly zero padding.  fp64 products: 561 lower tiles, more than
    the resident workgroups, so they run the stream-K kernel with split tiles;
    4112 (a multiple of 16) takes the DMA main loop, 4100 the register-staged
    one.  The oracle's eigendecomposition takes minutes at this size, so the
    input has a known spectrum instead: H = Q diag(lam) Q^T with Q orthogonal
    (Householder QR of a Gaussian matrix, LAPACK through numpy) and lam spread
    over [-1, 1], whose projection is Q diag(max(lam, 0)) Q^T exactly.
    Rounding H to fp32 moves the projection by at most ||H32 - H||_F (projection
    onto a convex set is non-expansive), about 6e-8 of ||P||_F here.  A second
    call on the same input must give the same bits (integer sums are exact;
    split fp64 tiles are summed in a fixed order whichever side finishes last)."""
    rng = np.random.default_rng(K)
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    lam = np.linspace(-1.0, 1.0, K)
    rng.shuffle(lam)
    H64 = (Q * lam) @ Q.T
    H64 = (H64 + H64.T) / 2
    P_exact = (Q * np.maximum(lam, 0.0)) @ Q.T
    H = H64.astype(np.float32)
    assert np.linalg.norm(H - H64) / np.linalg.norm(P_exact) < 1e-7
    gq.gq_set_psd_products(gq.GQ_PSD_F64 if kind == "f64" else gq.GQ_PSD_AUTO)
    try:
        P = _gpu_psd(gq, H)
        P2 = _gpu_psd(gq, H)
    finally:
        gq.gq_set_psd_products(gq.GQ_PSD_AUTO)
    assert np.array_equal(P, P.T)
    assert _relF(P, P_exact) < 1e-5
    assert np.array_equal(P2.view(np.uint32), P.view(np.uint32))


def test_psd_stored_hessian_full_size(gq, orc):
    """The stored-Hessian workload at its full size (K=1024): Gram -> bf16 tril
    storage -> unpack -> projection, both sides from the same stored matrix."""
    wl = g.WORKLOADS["stored1024"]
    X = g.x_chunk(wl)
    H32 = orc.gram(X).astype(np.float32)
    Hs = orc.unpack_tril(orc.pack_tril(H32), wl.K)
    P = _gpu_psd(gq, Hs)
    _, P64 = orc.psd_project(Hs, 1, return_f64=True)
    assert _relF(P, P64) < 1e-5
    assert np.array_equal(P, P.T)


def test_psd_keeps_psd_input_and_zero(gq, orc):
    wl = g.WORKLOADS["tiny"]
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    H = _sym(H).astype(np.float32)
    P = _gpu_psd(gq, H)
    assert _relF(P, H) < 1e-5
    Z = np.zeros((64, 64), np.float32)
    assert np.array_equal(_gpu_psd(gq, Z), Z)


def test_psd_rejects_nonfinite(gq):
    H = np.eye(40, dtype=np.float32)
    H[20, 3] = np.nan
    with pytest.raises(gq.GQError) as e:
        _gpu_psd(gq, H)
    assert e.value.status == gq.GQ_ERR_NONFINITE


# ------------------------------------------------------------------ factor U
def _gpu_U(gq, H, damp=0.01):
    K = H.shape[0]
    Ht = torch.from_numpy(np.ascontiguousarray(H, np.float32)).to(DEV)
    U = torch.empty(K, K, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_factor_workspace_size(K), DEV)
    gq.gptq_factor(U, Ht, damp, ws)
    return U.cpu().numpy()


@pytest.mark.parametrize("T,K", [(512, 128), (700, 200), (3000, 1024), (90, 64), (400, 66)])
def test_factor_matches_oracle(gq, orc, T, K):
    X = g.normal_matrix(T * 7 + K, g.S_X, T, K)
    H = orc.gram(X).astype(np.float32)
    U = _gpu_U(gq, H)
    st, Uo, mu = orc.gptq_U(H, 0.01)
    assert st == orc.OK
    assert np.all(np.tril(U, -1) == 0)
    assert _relF(U, Uo) < 1e-6


# ------------------------------------------------------------------ GPTQ
def _gpu_gptq(gq, W, H, G, damp=0.01, imp=None, want_qerr=True):
    N, K = W.shape
    Wt = torch.from_numpy(np.ascontiguousarray(W, np.float32)).to(DEV)
    Ht = torch.from_numpy(np.ascontiguousarray(H, np.float32)).to(DEV)
    it = None if imp is None else torch.from_numpy(np.ascontiguousarray(imp, np.float32)).to(DEV)
    codes = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(N, K // G, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_quantize_workspace_size(N, K, G), DEV)
    q = gq.gptq_quantize(codes, scales, Wt, Ht, it, G, damp, ws, want_qerr)
    return codes.cpu().numpy(), scales.cpu().numpy(), q


def _check_gptq(orc, W, H, G, codes_packed, scales, q, imp=None, damp=0.01):
    N, K = W.shape
    st, U, mu = orc.gptq_U(H, damp)
    assert st == orc.OK
    codes = orc.unpack_codes(codes_packed, K)
    oc, os_ = orc.gptq_sweep(W, U, G)
    ident = float((codes == oc).mean())
    rep = orc.gptq_replay(codes, scales, W, U, G)
    assert rep["inadmissible"] == 0, rep
    assert rep["scale_mismatch"] == 0, rep
    assert ident >= 0.999, (ident, rep)
    assert codes.min() >= -8 and codes.max() <= 7
    if q is not None:
        qo = orc.qerr(oc, os_, W, imp)
        assert abs(q - qo) / qo < 1e-4
        qg = orc.qerr(codes, scales, W, imp)          # the GPU's qerr of its own codes
        assert abs(q - qg) / qg < 1e-6
    return ident, rep


def test_gptq_tiny_workload(gq, orc):
    wl = g.WORKLOADS["tiny"]
    X = g.x_chunk(wl)
    W = g.weights(wl).numpy()
    H = orc.gram(X).astype(np.float32)
    imp = np.diag(H).copy()
    codes, scales, q = _gpu_gptq(gq, W, H, wl.group, wl.damp, imp)
    _check_gptq(orc, W, H, wl.group, codes, scales, q, imp)


@pytest.mark.parametrize("N,K,G", [(200, 256, 32), (33, 384, 128), (130, 200, 8), (64, 130, 2)])
def test_gptq_ragged_shapes(gq, orc, N, K, G):
    X = g.normal_matrix(N + K, g.S_X, 2 * K, K).numpy()
    mix = g.normal_matrix(N + K, g.S_A, K, K, 1.0 / np.sqrt(K)).numpy()
    X = (X @ (np.eye(K) + mix)).astype(np.float32)            # correlated channels
    H = orc.gram(X).astype(np.float32)
    W = g.uniform_weights(N + K, N, K).numpy()
    codes, scales, q = _gpu_gptq(gq, W, H, G)
    _check_gptq(orc, W, H, G, codes, scales, q)


def test_gptq_stored_workload_full_size(gq, orc):
    """Stored-Hessian workload at full size (N = K = 1024, G = 128): both sides
    quantise with the same projected Hessian."""
    wl = g.WORKLOADS["stored1024"]
    X = g.x_chunk(wl)
    H32 = orc.gram(X).astype(np.float32)
    Hs = orc.unpack_tril(orc.pack_tril(H32), wl.K)
    P = orc.psd_project(Hs)
    W = g.weights(wl).numpy()
    imp = np.diag(H32).copy()
    codes, scales, q = _gpu_gptq(gq, W, P, wl.group, wl.damp, imp)
    ident, rep = _check_gptq(orc, W, P, wl.group, codes, scales, q, imp)


def test_gptq_diagonal_hessian_is_rtn_bitwise(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = g.uniform_weights(5, 300, 512).numpy()
    d = np.exp(np.random.default_rng(0).standard_normal(512)).astype(np.float32)
    codes, scales, _ = _gpu_gptq(gq, W, np.diag(d), 64, 0.01, want_qerr=False)
    rc, rs = orc.rtn(W, 64)
    assert np.array_equal(orc.unpack_codes(codes, 512), rc)
    assert np.array_equal(scales, rs)


def _tiny_scale_weights():
    """Rows whose groups need the exact power-of-two guard of the quotient: a
    group of weights around 1e-30 (scale near 2^-102, where the correction
    step's remainder would underflow), a group of zeros and one subnormal value
    (a subnormal scale, whose reciprocal overflows), an all-subnormal group, and
    an ordinary group beside them."""
    rng = np.random.default_rng(7)
    W = np.zeros((4, 256), np.float32)
    W[:, 0:64] = (rng.uniform(-1, 1, (4, 64)) * 1e-30).astype(np.float32)
    W[:, 64:128] = 0.0
    W[:, 64 + 5] = np.float32(3e-39)                  # subnormal
    W[1, 64 + 9] = np.float32(-2e-39)
    W[:, 128:192] = (rng.uniform(-1, 1, (4, 64)) * 1e-39).astype(np.float32)
    W[:, 192:256] = rng.uniform(-1, 1, (4, 64)).astype(np.float32)
    return W


@pytest.mark.parametrize("flags", [0, 1])
def test_gptq_tiny_scales_are_rtn_bitwise(gq, orc, flags):
    """Diagonal H reduces GPTQ to round to nearest bit for bit also where the
    scale is tiny or subnormal.  The expected codes are checked on the CPU first:
    the subnormal value is the group's maximum, so it takes code 7 and the zeros
    beside it take 0; the 1e-30 group spans the whole grid."""
    W = _tiny_scale_weights()
    rc, rs = orc.rtn(W, 64)
    assert (rs[:, 1] > 0).all() and (rs[:, 1] < np.float32(1.2e-38)).all()     # subnormal scales
    assert (rc[:, 64 + 5] == 7).all() and (rc[0, 64:128][np.arange(64) != 5] == 0).all()
    assert rc[:, 0:64].min() == -7 and rc[:, 0:64].max() == 7
    assert (rs[:, 0] < 2.0 ** -60).all()
    d = np.exp(np.random.default_rng(1).standard_normal(256)).astype(np.float32)
    if flags:
        codes, scales, _ = _gpu_gptq_ex(gq, W, np.diag(d), 64, flags)
    else:
        codes, scales, _ = _gpu_gptq(gq, W, np.diag(d), 64, 0.01, want_qerr=False)
    assert np.array_equal(scales, rs)
    assert np.array_equal(orc.unpack_codes(codes, 256), rc)


def _gpu_gptq_ex(gq, W, H, G, flags, damp=0.01):
    N, K = W.shape
    c = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    s = torch.empty(N, K // G, dtype=torch.float32, device=DEV)
    ws = gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, flags), DEV)
    q = gq.gptq_quantize_ex(c, s, torch.from_numpy(W).to(DEV), torch.from_numpy(H).to(DEV), None, G, damp,
                            flags, ws, want_qerr=False)
    return c.cpu().numpy(), s.cpu().numpy(), q


def test_gptq_qerr_request_leaves_codes_identical(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    a = _gpu_gptq(gq, W, H, 32, want_qerr=True, imp=np.diag(H).copy())
    b = _gpu_gptq(gq, W, H, 32, want_qerr=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and b[2] is None
    c = _gpu_gptq(gq, W, H, 32, want_qerr=True, imp=np.diag(H).copy())
    assert c[2] == a[2]                                   # deterministic


def test_gptq_status_codes(gq, orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = orc.gram(g.x_chunk(wl)).astype(np.float32)
    cases = []
    W2 = W.copy(); W2[3, 7] = np.nan
    cases.append((W2, H, 32, gq.GQ_ERR_NONFINITE))
    H2 = H.copy(); H2[9, 2] = np.inf
    cases.append((W, H2, 32, gq.GQ_ERR_NONFINITE))
    cases.append((W, np.zeros_like(H), 32, gq.GQ_ERR_NO_CALIBRATION))
    Hi = np.eye(128, dtype=np.float32); Hi[127, 127] = -50.0
    cases.append((W, Hi, 32, gq.GQ_ERR_NOT_PD))
    cases.append((W, H, 48, gq.GQ_ERR_INVALID_ARG))
    for Wc, Hc, G, want in cases:
        with pytest.raises(gq.GQError) as e:
            _gpu_gptq(gq, Wc, Hc, G)
        assert e.value.status == want
        # the oracle agrees on the same inputs
        assert orc.gptq(Wc, Hc, G)[0] == want
    H3 = H.copy(); H3[2, 9] = np.nan                   # upper triangle is never read
    _gpu_gptq(gq, W, H3, 32)
