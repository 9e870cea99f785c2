"""CPU reference (oracle) for the calibration-Hessian GPTQ path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The product library never imports it, and it
shares no code with the HIP path.  The arithmetic lives in `gq_oracle.c`
(plain fp64 C, OpenMP over independent rows); this file only marshals numpy
arrays through ctypes and builds the shared object with gcc.

Parity is pinned for every function by the CPU tests (tests/test_oracle_*.py)
against brute force, closed forms, invariants, library special cases and the
values the pages print.  GPTQ codes on correlated Hessians at K >= 1024 are
"parity unpinned" beyond those invariants: the pages publish no golden codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gq_oracle.c")
_LIB = os.path.join(_HERE, "libgq_oracle.so")

OK, ERR_INVALID_ARG, ERR_NOT_PD, ERR_NONFINITE, ERR_NO_CALIBRATION = 0, 1, 2, 3, 4
ERR_NO_CONVERGENCE = 6


def build(force: bool = False) -> str:
    """Compile gq_oracle.c into libgq_oracle.so (portable x86-64, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_mutant(mutant: int, outdir: str) -> str:
    """Compile a deliberately wrong variant (-DORC_MUTANT=n) for the mutation tests."""
    out = os.path.join(outdir, f"libgq_oracle_mutant{mutant}.so")
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", f"-DORC_MUTANT={mutant}", _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def use_library(path):
    """Point this module at another build of gq_oracle.c (mutation tests); None restores."""
    global _lib
    _lib = None if path is None else _load(path)


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = _load(_LIB)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    I = ctypes.c_int
    sig = {
        "orc_num_threads": (I, []),
        "orc_gram_accumulate": (None, [P, P, I64, I64]),
        "orc_gram_entries": (None, [P, P, I64, I64, P, P, I64]),
        "orc_tril_bytes": (I64, [I64]),
        "orc_pack_tril": (None, [P, P, I64]),
        "orc_unpack_tril": (None, [P, P, I64]),
        "orc_eigh_jacobi": (I, [P, P, P, I64, I]),
        "orc_eigh_tridiag": (I, [P, P, P, I64]),
        "orc_eigh": (I, [P, P, P, I64, I]),
        "orc_eigvalsh": (I, [P, P, I64]),
        "orc_eigvalsh_f64": (I, [P, P, I64]),
        "orc_psd_project": (I, [P, P, P, I64, I]),
        "orc_cholesky_lower": (I, [P, I64]),
        "orc_diag_mean": (D, [P, I64]),
        "orc_gptq_U": (I, [P, P, I64, D, P]),
        "orc_gptq_sweep": (None, [P, P, P, P, I64, I64, P, I64]),
        "orc_rtn": (None, [P, P, P, I64, I64, I64]),
        "orc_qerr": (D, [P, P, P, P, I64, I64, I64, P]),
        "orc_pack_codes": (None, [P, P, I64, I64]),
        "orc_unpack_codes": (None, [P, P, I64, I64]),
        "orc_gptq": (I, [P, P, P, P, P, P, I64, I64, I64, D]),
        "orc_gptq_replay": (None, [P, P, P, P, P, P, I64, I64, P, I64, D, D]),
        "orc_gptq_sweep_ex": (None, [P, P, P, P, I64, I64, P, I64, I, P]),
        "orc_rtn_ex": (None, [P, P, P, I64, I64, I64, I, P]),
        "orc_qerr_ex": (D, [P, P, P, P, I64, I64, I64, P, P]),
        "orc_gptq_ex": (I, [P, P, P, P, P, P, I64, I64, I64, D, I, P]),
        "orc_gptq_replay_ex": (None, [P, P, P, P, P, P, I64, I64, P, I64, D, D, I, P]),
        "orc_gptq_sweep_gx": (None, [P, P, P, P, I64, I64, P, I64, I, P, P]),
        "orc_gptq_replay_gx": (None, [P, P, P, P, P, P, I64, I64, P, I64, D, D, I, P, P]),
        "orc_gptq_replay_hx": (None, [P, P, P, P, P, P, I64, I64, P, I64, D, D, I, P, P, P]),
        "orc_act_order_perm": (None, [P, P, I64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _np(x, dtype):
    """Accept numpy arrays or torch tensors (CPU; bf16 is widened exactly to fp32)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.to(torch.float32)
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return _c(x, dtype)


class OracleError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def num_threads() -> int:
    return lib().orc_num_threads()


# ------------------------------------------------------------------ Gram
def gram(X, H=None):
    """fp64 H (+)= X^T X for X (T x K, fp32 or bf16 values)."""
    X = _np(X, np.float32)
    T, K = X.shape
    if H is None:
        H = np.zeros((K, K), np.float64)
    lib().orc_gram_accumulate(_p(H), _p(X), T, K)
    return H


def gram_entries(X, I, J):
    X = _np(X, np.float32)
    T, K = X.shape
    I = _c(I, np.int64)
    J = _c(J, np.int64)
    out = np.zeros(len(I), np.float64)
    lib().orc_gram_entries(_p(out), _p(X), T, K, _p(I), _p(J), len(I))
    return out


# ------------------------------------------------------------------ tril storage
def tril_bytes(K: int) -> int:
    return int(lib().orc_tril_bytes(K))


def pack_tril(H):
    H = _np(H, np.float32)
    K = H.shape[0]
    blob = np.zeros(tril_bytes(K), np.uint8)
    lib().orc_pack_tril(_p(blob), _p(H), K)
    return blob


def unpack_tril(blob, K: int):
    blob = _c(blob, np.uint8)
    assert blob.size == tril_bytes(K)
    H = np.zeros((K, K), np.float32)
    lib().orc_unpack_tril(_p(H), _p(blob), K)
    return H


# ------------------------------------------------------------------ eigen / PSD
def eigh(H, method: int = 1):
    """(w, V) with V[:, k] the eigenvector of w[k]; method 0 Jacobi, 1 tridiagonal QR."""
    H = _np(H, np.float32)
    K = H.shape[0]
    w = np.zeros(K, np.float64)
    Vt = np.zeros((K, K), np.float64)
    st = lib().orc_eigh(_p(w), _p(Vt), _p(H), K, method)
    if st:
        raise OracleError(st, "eigh")
    return w, Vt.T.copy()


def eigvalsh(H):
    H = _np(H, np.float32)
    K = H.shape[0]
    w = np.zeros(K, np.float64)
    st = lib().orc_eigvalsh(_p(w), _p(H), K)
    if st:
        raise OracleError(st, "eigvalsh")
    return np.sort(w)


def eigvalsh_f64(S):
    S = _c(S, np.float64)
    K = S.shape[0]
    w = np.zeros(K, np.float64)
    st = lib().orc_eigvalsh_f64(_p(w), _p(S), K)
    if st:
        raise OracleError(st, "eigvalsh_f64")
    return np.sort(w)


def psd_project(H, method: int = 1, return_f64: bool = False):
    H = _np(H, np.float32)
    K = H.shape[0]
    P = np.zeros((K, K), np.float32)
    P64 = np.zeros((K, K), np.float64) if return_f64 else None
    st = lib().orc_psd_project(_p(P), _p(P64), _p(H), K, method)
    if st:
        raise OracleError(st, "psd_project")
    return (P, P64) if return_f64 else P


# ------------------------------------------------------------------ GPTQ
def cholesky_lower(A):
    A = _c(A, np.float64).copy()
    st = lib().orc_cholesky_lower(_p(A), A.shape[0])
    return st, A


def diag_mean(H) -> float:
    H = _np(H, np.float32)
    return float(lib().orc_diag_mean(_p(H), H.shape[0]))


def gptq_U(H, damp: float = 0.01):
    """(status, U fp64 upper, mu) with (H + damp*mu*I)^-1 = U^T U."""
    H = _np(H, np.float32)
    K = H.shape[0]
    U = np.zeros((K, K), np.float64)
    mu = ctypes.c_double(0.0)
    st = lib().orc_gptq_U(_p(U), _p(H), K, damp, ctypes.byref(mu))
    return st, U, mu.value


def gptq_U_lapack(H, damp: float = 0.01):
    """The same U as gptq_U, by the same literal route, for sizes where the plain
    C loops take minutes (K = 17408): L = chol(H_d), H_d^-1 = L^-T L^-1, U = the
    upper Cholesky factor of H_d^-1, with H_d = H + damp * mean(diag H) * I read
    from H's lower triangle (ork-driver wiki "Exp 2026-08-18 GPTQ Int4":
    Cholesky-based Hessian inverse; hipfire-calib-data "The fix": damping in units
    of mean(diag H)).  Each step is one LAPACK primitive through torch's CPU
    backend in fp64 (potrf, potri, potrf); statuses as gptq_U.  Pinned to gptq_U
    in tests/test_oracle_gptq.py.  Returns (status, U fp64 upper, mu)."""
    import torch
    H = _np(H, np.float32)
    K = H.shape[0]
    low = np.tril(H)
    if not np.isfinite(low).all():
        return ERR_NONFINITE, None, float("nan")
    mu = float(np.diag(H).astype(np.float64).sum() / K)
    if not mu > 0.0:
        return ERR_NO_CALIBRATION, None, mu
    A = torch.from_numpy(low.astype(np.float64))
    A = A + torch.tril(A, -1).T
    A.diagonal().add_(damp * mu)
    L, info = torch.linalg.cholesky_ex(A)
    del A
    if int(info) != 0:
        return ERR_NOT_PD, None, mu
    Hinv = torch.cholesky_inverse(L)          # (L L^T)^-1 = L^-T L^-1
    del L
    Lh, info = torch.linalg.cholesky_ex(Hinv)
    del Hinv
    if int(info) != 0:
        return ERR_NOT_PD, None, mu
    return OK, Lh.T.contiguous().numpy(), mu


# Sweep and pack switches (gq_oracle.c): scales fixed from the original weights
# before the sweep; the NF4 codebook instead of the uniform int4 grid.
STATIC_GROUPS = 1
NF4 = 2
ACT_ORDER = 4          # with STATIC_GROUPS: columns by decreasing diag(H) (gq_oracle.c)

_NF4 = None


def nf4_levels():
    """The 16 NF4 levels as fp32, ascending (QLoRA, Dettmers et al. 2023, the
    4-bit NormalFloat data type): quantiles of the standard normal at evenly
    spaced probabilities, 8 on the positive side and 7 on the negative side so
    that 0 is a level, the outermost probability 1 - d with d = (1/32 + 1/30)/2
    (the mean of the half-bin widths of 16 and 15 bins) so that it stays finite,
    then scaled to [-1, 1] by the largest.  The quantile function is scipy's."""
    global _NF4
    if _NF4 is None:
        from scipy.stats import norm
        d = 0.5 * (1.0 / 32 + 1.0 / 30)
        pos = norm.ppf(np.linspace(1.0 - d, 0.5, 9)[:-1])
        neg = -norm.ppf(np.linspace(1.0 - d, 0.5, 8)[:-1])
        L = np.sort(np.concatenate([neg, [0.0], pos]))
        _NF4 = (L / pos.max()).astype(np.float32)
    return _NF4.copy()


def _book(flags):
    return nf4_levels() if flags & NF4 else None


def act_order_perm(H):
    """perm[a] = the column with the a-th largest diagonal entry of H (fp32),
    equal entries in increasing column order."""
    H = _np(H, np.float32)
    K = H.shape[0]
    perm = np.zeros(K, np.int64)
    lib().orc_act_order_perm(_p(perm), _p(H), K)
    return perm


def gptq_sweep(W, U, G: int, rows=None, flags: int = 0, gidx=None):
    """Codes (len(rows) x K int8: signed int4, or NF4 level indices) and scales of
    the GPTQ sweep of W's rows under U.  gidx (static groups only): the group of
    each column in this order, when not contiguous (act order)."""
    W = _np(W, np.float32)
    U = _c(U, np.float64)
    N, K = W.shape
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    codes = np.zeros((len(rows), K), np.int8)
    scales = np.zeros((len(rows), K // G), np.float32)
    gidx = None if gidx is None else _c(gidx, np.int64)
    lib().orc_gptq_sweep_gx(_p(codes), _p(scales), _p(W), _p(U), K, G, _p(rows), len(rows), flags,
                            _p(_book(flags)), _p(gidx))
    return codes, scales


def rtn(W, G: int, flags: int = 0):
    W = _np(W, np.float32)
    N, K = W.shape
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // G), np.float32)
    lib().orc_rtn_ex(_p(codes), _p(scales), _p(W), N, K, G, flags, _p(_book(flags)))
    return codes, scales


def qerr(codes, scales, W, imp=None, return_sums: bool = False, flags: int = 0):
    W = _np(W, np.float32)
    N, K = W.shape
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    G = K // scales.shape[1]
    imp = None if imp is None else _np(imp, np.float32)
    nd = np.zeros(2, np.float64)
    q = float(lib().orc_qerr_ex(_p(codes), _p(scales), _p(W), _p(imp), N, K, G, _p(_book(flags)), _p(nd)))
    return (q, nd) if return_sums else q


def pack_codes(codes):
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.zeros((N, K // 2), np.uint8)
    lib().orc_pack_codes(_p(out), _p(codes), N, K)
    return out


def unpack_codes(packed, K: int, flags: int = 0):
    """Codes from two nibbles per byte (column 2m low): signed int4, or with NF4
    the unsigned level indices 0..15."""
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    codes = np.zeros((N, K), np.int8)
    lib().orc_unpack_codes(_p(codes), _p(packed), N, K)
    if flags & NF4:
        codes = (codes & 0xF).astype(np.int8)
    return codes


def gptq(W, H, G: int, damp: float = 0.01, imp=None, want_qerr: bool = True, flags: int = 0):
    """(status, codes int8 N x K, scales N x K/G, qerr or None)."""
    W = _np(W, np.float32)
    H = _np(H, np.float32)
    N, K = W.shape
    imp = None if imp is None else _np(imp, np.float32)
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, max(1, K // max(G, 1))), np.float32)
    q = ctypes.c_double(0.0)
    st = lib().orc_gptq_ex(_p(codes), _p(scales), ctypes.byref(q) if want_qerr else None,
                           _p(W), _p(H), _p(imp), N, K, G, damp, flags, _p(_book(flags)))
    return st, codes, scales, (q.value if want_qerr else None)


def gptq_replay(cand_codes, cand_scales, W, U, G: int, rows=None, delta: float = 1e-3,
                scale_tol: float = 1e-5, flags: int = 0, gidx=None):
    """Admissibility of candidate codes/scales for W's listed rows (see gq_oracle.c).
    flip_gap_hist counts the accepted tie flips by their distance from the exact
    tie, in steps: [0, 1e-7), [1e-7, 1e-6), [1e-6, 1e-5), [1e-5, 1e-4),
    [1e-4, 1e-3), [1e-3, delta]."""
    W = _np(W, np.float32)
    U = _c(U, np.float64)
    N, K = W.shape
    rows = np.arange(N, dtype=np.int64) if rows is None else _c(rows, np.int64)
    cc = _c(cand_codes, np.int8)
    cs = _c(cand_scales, np.float32)
    assert cc.shape == (len(rows), K) and cs.shape == (len(rows), K // G)
    stats = np.zeros(4, np.int64)
    hist = np.zeros(6, np.int64)
    mrel = ctypes.c_double(0.0)
    gidx = None if gidx is None else _c(gidx, np.int64)
    lib().orc_gptq_replay_hx(_p(stats), ctypes.byref(mrel), _p(cc), _p(cs), _p(W), _p(U), K, G,
                             _p(rows), len(rows), delta, scale_tol, flags, _p(_book(flags)), _p(gidx),
                             _p(hist))
    return {"exact": int(stats[0]), "tie_flips": int(stats[1]), "inadmissible": int(stats[2]),
            "scale_mismatch": int(stats[3]), "max_scale_rel": mrel.value,
            "flip_gap_hist": [int(x) for x in hist]}


# ------------------------------------------------------------------ Hadamard rotation
def sylvester_hadamard(b: int):
    """H_b by Sylvester's doubling: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]
    (the rotation GPTQ composes with, ork-driver wiki "Exp 2026-08-18 GPTQ Int4")."""
    if b < 1 or b & (b - 1):
        raise ValueError("b must be a power of two")
    Hm = np.ones((1, 1))
    while Hm.shape[0] < b:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def hadamard_rotation(K: int, b: int, signs=None):
    """R = blockdiag(H_b, ..., H_b) diag(signs) / sqrt(b), K x K, fp64."""
    if K % b:
        raise ValueError("b must divide K")
    Hb = sylvester_hadamard(b) / np.sqrt(b)
    R = np.kron(np.eye(K // b), Hb)
    if signs is not None:
        R = R * np.asarray(signs, np.float64)[None, :]
    return R


def hadamard_rotate_rows(A, b: int, signs=None):
    """A R^T in fp64 (each row rotated), returned as fp32."""
    A = np.asarray(A, np.float64)
    R = hadamard_rotation(A.shape[1], b, signs)
    return (A @ R.T).astype(np.float32)


def hadamard_rotate_hessian(H, b: int, signs=None):
    """R H R^T in fp64, returned as fp32."""
    H = np.asarray(H, np.float64)
    R = hadamard_rotation(H.shape[0], b, signs)
    return (R @ H @ R.T).astype(np.float32)

