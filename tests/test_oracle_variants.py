"""Pins of the oracle's GPTQ variants: static groups (every scale fixed before the
sweep from the original weights) and the NF4 codebook (the 4-bit pack the
ork-driver wiki's qerr section scores beside the uniform grid, "Exp 2026-08-18
GPTQ Int4": 0.0936 on uniformly distributed weights).

What fixes them from outside the oracle:
  - the NF4 table's shape (16 levels in [-1, 1], 0 exact, 7 below and 8 above);
  - the wiki's NF4 qerr on uniform weights, and the exact integral of the squared
    rounding error over the table's cells (no sampling), scaled to groups of G;
  - nearest-level codes by brute force (argmin over the 16 levels);
  - static groups: scales equal to the round-to-nearest scales bit for bit, and
    a diagonal Hessian reducing every variant to round-to-nearest;
  - an independent OBQ recursion (freshly inverted Hessians of the columns not yet
    quantised) carrying each variant's scale rule and grid;
  - act order (AutoGPTQ's desc_act, with static groups): the permutation against
    numpy's stable argsort, the OBQ recursion run in that column order with each
    column's original group's scale, and the identity permutation when the
    diagonal already decreases.
"""
import json
import math
import os

import numpy as np
import pytest

import synthgen as g

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gram32(orc, X):
    H = orc.gram(X)
    return (np.tril(H) + np.tril(H, -1).T).astype(np.float32)


def test_nf4_table_shape(orc):
    L = orc.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L[0] == -1.0 and L[7] == 0.0 and L[15] == 1.0
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8
    # finer near zero, where normal weights are dense: spacing grows outwards
    d = np.diff(L)
    assert np.all(np.diff(d[7:]) > 0) and np.all(np.diff(d[:7]) < 0)


def _nf4_cell_mse(L):
    """E[(x - L(x))^2] for x uniform on (-1, 1), L(x) the nearest level: the exact
    integral over each level's cell between the midpoints."""
    L = np.asarray(L, np.float64)
    edges = np.concatenate([[-1.0], (L[:-1] + L[1:]) / 2, [1.0]])
    tot = 0.0
    for c in range(16):
        a, b = edges[c] - L[c], edges[c + 1] - L[c]
        tot += (b ** 3 - a ** 3) / 3.0
    return tot / 2.0


def test_nf4_qerr_on_uniform_weights(orc):
    """The group maximum lands on +-1 exactly; the other G - 1 values of a group,
    divided by the maximum M, are uniform on (-1, 1), and E[M^2] = G/(G+2), so
    qerr = sqrt(3 E_cell (G-1)/(G+2)).  Its large-G limit is the wiki's 0.0936."""
    gold = json.load(open(os.path.join(GOLD, "pages_values.json")))["qerr_nf4"]
    L = orc.nf4_levels()
    e = _nf4_cell_mse(L)
    limit = math.sqrt(3 * e)
    assert limit == pytest.approx(gold["summary"], rel=0.004)
    assert limit == pytest.approx(gold["measured"], rel=0.004)
    W = g.uniform_weights(8, 1024, 1024).numpy()            # 2^20 weights
    for G in (16, 128, 1024):
        codes, scales = orc.rtn(W, G, flags=orc.NF4)
        q = orc.qerr(codes, scales, W, flags=orc.NF4)
        assert q == pytest.approx(limit * math.sqrt((G - 1) / (G + 2)), rel=0.01), G
        cu, su = orc.rtn(W, G)
        assert orc.qerr(cu, su, W) < q                         # the uniform grid fits uniform data better
    codes, scales = orc.rtn(W, 1024, flags=orc.NF4)
    assert orc.qerr(codes, scales, W, flags=orc.NF4) == pytest.approx(gold["measured"], rel=0.004)


def test_nf4_codes_are_nearest_levels(orc):
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    W[3, 32:64] = 0.0                                         # an all-zero group
    G = 32
    codes, scales = orc.rtn(W, G, flags=orc.NF4)
    L = orc.nf4_levels().astype(np.float64)
    amax = np.abs(W.reshape(64, -1, G)).max(-1)
    assert np.array_equal(scales, amax.astype(np.float32))    # scale = absmax, no division
    s = np.repeat(scales, G, axis=1)
    x = np.where(s > 0, W / np.where(s > 0, s, 1), 0).astype(np.float32).astype(np.float64)
    dist = np.abs(x[..., None] - L)
    want = dist.argmin(-1)
    srt = np.sort(dist, -1)
    clear = srt[..., 1] - srt[..., 0] > 1e-6                   # not at a midpoint
    assert clear.mean() > 0.99
    assert np.array_equal(codes[clear], want[clear])
    assert np.all(codes[3, 32:64] == 7) and scales[3, 1] == 0.0   # level 0.0
    # each group's extreme value is reproduced exactly
    n = np.arange(64)[:, None]
    k = np.abs(W.reshape(64, -1, G)).argmax(-1) + np.arange(0, 256, G)[None, :]
    assert np.array_equal(np.abs(L[codes[n, k]] * scales), np.abs(W[n, k]))


def _obq(W, H, G, damp, static=False, book=None):
    """Sequential OBQ with freshly inverted Hessians of the remaining columns
    (numpy LAPACK), any scale rule and grid: uniform clamp(rint(v), -8, 7) with
    scale absmax/7, or the codebook's nearest level by argmin with scale absmax."""
    W0 = W.astype(np.float64)
    W = W0.copy()
    N, K = W.shape
    Hd = H.astype(np.float64)
    Hd = Hd + damp * np.trace(Hd) / K * np.eye(K)
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // G), np.float32)
    Lb = None if book is None else np.asarray(book, np.float64)
    s = np.zeros(N, np.float32)
    for i in range(K):
        Finv = np.linalg.inv(Hd[i:, i:])
        if i % G == 0:
            src = W0 if static else W
            m = np.abs(src[:, i:i + G]).max(1).astype(np.float32)
            s = m if Lb is not None else (m / np.float32(7)).astype(np.float32)
            scales[:, i // G] = s
        v = np.where(s > 0, W[:, i].astype(np.float32) / np.where(s > 0, s, 1), 0).astype(np.float32)
        if Lb is None:
            c = np.clip(np.rint(v), -8, 7)
            q = c * s.astype(np.float64)
        else:
            c = np.abs(v.astype(np.float64)[:, None] - Lb).argmin(1)
            q = Lb[c] * s.astype(np.float64)
        codes[:, i] = c
        err = (W[:, i] - q) / Finv[0, 0]
        W[:, i:] -= np.outer(err, Finv[0, :])
    return codes, scales


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_variants_equal_obq_recursion(orc, flags):
    rng = np.random.default_rng(12)
    N, K, G = 24, 48, 16
    X = (rng.standard_normal((160, 12)) @ rng.standard_normal((12, K)) +
         0.3 * rng.standard_normal((160, K))).astype(np.float32)
    H = _gram32(orc, X)
    W = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=flags)
    assert st == orc.OK
    rc, rs = _obq(W, H, G, 0.01, static=bool(flags & orc.STATIC_GROUPS),
                  book=orc.nf4_levels() if flags & orc.NF4 else None)
    assert np.array_equal(codes, rc)
    np.testing.assert_allclose(scales, rs, rtol=1e-6)


def test_static_groups_scales_are_rtn_scales(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    for book_flag in (0, orc.NF4):
        st, codes, scales, _ = orc.gptq(W, H, wl.group, 0.01, flags=orc.STATIC_GROUPS | book_flag)
        assert st == orc.OK
        _, rs = orc.rtn(W, wl.group, flags=book_flag)
        assert np.array_equal(scales, rs)
        # the dynamic sweep's scales differ once feedback has moved the values
        _, _, dyn, _ = orc.gptq(W, H, wl.group, 0.01, flags=book_flag)
        assert not np.array_equal(dyn, rs)


def test_diagonal_hessian_reduces_every_variant_to_rtn(orc):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()
    H = _gram32(orc, g.x_chunk(wl))
    Hd = np.diag(np.diag(H)).astype(np.float32)
    for flags in (0, 1, 2, 3):
        st, codes, scales, q = orc.gptq(W, Hd, wl.group, 0.01, flags=flags)
        rc, rs = orc.rtn(W, wl.group, flags=flags & orc.NF4)
        assert st == orc.OK and np.array_equal(codes, rc) and np.array_equal(scales, rs), flags
        assert q == orc.qerr(rc, rs, W, flags=flags & orc.NF4)


def test_static_zero_group_still_feeds_back(orc):
    """A group that is all zero in the original weights has scale 0 under static
    groups; error feedback may still move its values, which then round to the
    zero code and pass their whole value on."""
    rng = np.random.default_rng(8)
    K, G = 8, 4
    X = rng.standard_normal((64, K)).astype(np.float32)
    X[:, 4:] += X[:, :4]                                        # couple the two groups
    H = _gram32(orc, X)
    W = rng.uniform(-1, 1, (6, K)).astype(np.float32)
    W[:, 4:] = 0.0
    for book_flag in (0, orc.NF4):
        flags = orc.STATIC_GROUPS | book_flag
        st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=flags)
        assert np.all(scales[:, 1] == 0.0)
        assert np.all(codes[:, 4:] == (7 if book_flag else 0))
        rc, rs = _obq(W, H, G, 0.01, static=True, book=orc.nf4_levels() if book_flag else None)
        assert np.array_equal(codes, rc)


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_replay_accepts_own_codes_and_rejects_others(orc, flags):
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()[:32]
    H = _gram32(orc, g.x_chunk(wl))
    st, U, _ = orc.gptq_U(H, 0.01)
    codes, scales = orc.gptq_sweep(W, U, wl.group, flags=flags)
    rep = orc.gptq_replay(codes, scales, W, U, wl.group, flags=flags)
    assert rep["inadmissible"] == 0 and rep["scale_mismatch"] == 0 and rep["tie_flips"] == 0
    assert rep["exact"] == codes.size
    bad = codes.copy()
    hi = 15 if flags & orc.NF4 else 7
    bad[5, 40] = bad[5, 40] - 2 if bad[5, 40] >= 2 - (0 if flags & orc.NF4 else 8) else bad[5, 40] + 2
    assert 0 <= bad[5, 40] + (0 if flags & orc.NF4 else 8) <= hi + (0 if flags & orc.NF4 else 8)
    rep = orc.gptq_replay(bad, scales, W, U, wl.group, flags=flags)
    assert rep["inadmissible"] >= 1


def test_nf4_pack_roundtrip(orc):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (5, 64)).astype(np.int8)
    packed = orc.pack_codes(codes)
    assert np.array_equal(orc.unpack_codes(packed, 64, flags=orc.NF4), codes)
    assert np.array_equal(packed[:, 0] & 0xF, codes[:, 0].astype(np.uint8))


# ------------------------------------------------------------------ act order
def _obq_order(W, H, G, damp, perm, book=None):
    """OBQ (freshly inverted Hessians of the remaining columns) taking the columns
    in the order perm, each with the static scale of its original contiguous group
    (absmax of the original weights; /7 on the uniform grid); codes returned in
    the original column order."""
    W0 = W.astype(np.float64)
    N, K = W.shape
    Hs = H.astype(np.float64)
    Hd = Hs + damp * np.trace(Hs) / K * np.eye(K)
    Hp = Hd[np.ix_(perm, perm)]
    Wp = W0[:, perm].copy()
    Lb = None if book is None else np.asarray(book, np.float64)
    amax = np.abs(W0).reshape(N, -1, G).max(-1).astype(np.float32)
    stab = amax if Lb is not None else (amax / np.float32(7)).astype(np.float32)
    cp = np.zeros((N, K), np.int8)
    for a in range(K):
        Finv = np.linalg.inv(Hp[a:, a:])
        s = stab[:, perm[a] // G]
        v = np.where(s > 0, Wp[:, a].astype(np.float32) / np.where(s > 0, s, 1), 0).astype(np.float32)
        if Lb is None:
            c = np.clip(np.rint(v), -8, 7)
            q = c * s.astype(np.float64)
        else:
            c = np.abs(v.astype(np.float64)[:, None] - Lb).argmin(1)
            q = Lb[c] * s.astype(np.float64)
        cp[:, a] = c
        err = (Wp[:, a] - q) / Finv[0, 0]
        Wp[:, a:] -= np.outer(err, Finv[0, :])
    codes = np.zeros_like(cp)
    codes[:, perm] = cp
    return codes, stab


def test_act_order_permutation(orc):
    rng = np.random.default_rng(21)
    K = 40
    X = (rng.standard_normal((100, K)) * rng.uniform(0.2, 3.0, K)).astype(np.float32)
    H = _gram32(orc, X)
    H[5, 5] = H[9, 9] = H[30, 30] = H[2, 2]                   # ties, kept in column order
    perm = orc.act_order_perm(H)
    assert np.array_equal(perm, np.argsort(-np.diag(H), kind="stable"))
    d = np.diag(H)[perm]
    assert np.all(d[:-1] >= d[1:])


@pytest.mark.parametrize("book_flag", [0, 2])
def test_act_order_equals_obq_in_that_order(orc, book_flag):
    rng = np.random.default_rng(13)
    N, K, G = 20, 48, 16
    X = (rng.standard_normal((160, 12)) @ rng.standard_normal((12, K)) +
         0.3 * rng.standard_normal((160, K))).astype(np.float32)
    X *= rng.uniform(0.3, 3.0, K).astype(np.float32)            # a spread of channel energies
    H = _gram32(orc, X)
    W = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    flags = orc.STATIC_GROUPS | orc.ACT_ORDER | book_flag
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=flags)
    assert st == orc.OK
    perm = np.argsort(-np.diag(H), kind="stable")
    assert not np.array_equal(perm, np.arange(K))
    rc, rs = _obq_order(W, H, G, 0.01, perm, orc.nf4_levels() if book_flag else None)
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales, rs)
    # and it differs from the natural order
    _, c0, _, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=orc.STATIC_GROUPS | book_flag)
    assert not np.array_equal(codes, c0)


def test_act_order_with_sorted_diagonal_is_static(orc):
    """A Hessian whose diagonal already decreases gives the identity permutation,
    so act order changes nothing."""
    rng = np.random.default_rng(14)
    K, G = 64, 16
    C = orc.gram(rng.standard_normal((200, K)).astype(np.float32))
    C = C / np.sqrt(np.outer(np.diag(C), np.diag(C)))          # unit diagonal
    D = np.linspace(3.0, 0.5, K)
    H = (D[:, None] * C * D[None, :]).astype(np.float32)       # diagonal D^2, decreasing
    assert np.all(np.diff(np.diag(H)) < 0)
    W = rng.uniform(-1, 1, (12, K)).astype(np.float32)
    for book_flag in (0, orc.NF4):
        a = orc.gptq(W, H, G, 0.01, flags=orc.STATIC_GROUPS | orc.ACT_ORDER | book_flag)
        b = orc.gptq(W, H, G, 0.01, flags=orc.STATIC_GROUPS | book_flag)
        assert a[0] == b[0] == orc.OK
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and a[3] == b[3]


def test_act_order_needs_static_groups(orc):
    W = np.ones((2, 8), np.float32)
    H = np.eye(8, dtype=np.float32)
    st, *_ = orc.gptq(W, H, 4, 0.01, flags=orc.ACT_ORDER)
    assert st == orc.ERR_INVALID_ARG


def test_replay_with_group_map(orc):
    """The replay on the permuted problem (W and H permuted, each column's original
    group as its group) accepts act order's codes put in that order."""
    wl = g.WORKLOADS["tiny"]
    W = g.weights(wl).numpy()[:24]
    H = _gram32(orc, g.x_chunk(wl))
    G = wl.group
    flags = orc.STATIC_GROUPS | orc.ACT_ORDER
    st, codes, scales, _ = orc.gptq(W, H, G, 0.01, want_qerr=False, flags=flags)
    perm = orc.act_order_perm(H)
    Hp = H[np.ix_(perm, perm)]
    st, Up, _ = orc.gptq_U(Hp, 0.01)
    rep = orc.gptq_replay(codes[:, perm], scales, W[:, perm], Up, G, flags=orc.STATIC_GROUPS, gidx=perm // G)
    assert rep["exact"] == codes.size and rep["scale_mismatch"] == 0
