"""Python binding of libgq.so, the calibration-Hessian GPTQ int4 library for MI355X.

Thin ctypes marshalling over the C ABI declared in include/gq.h: each function
takes torch tensors that already live on the GPU, passes their device pointers
and the current HIP stream, and raises GQError on a non-zero status.  Every step
of the path runs in the library's HIP kernels; nothing here computes.  PyTorch
supplies device memory and streams only.  The library must be built
(``python -m post_weight_quantization_accumulate_amd.build``); there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

(GQ_OK, GQ_ERR_INVALID_ARG, GQ_ERR_NOT_PD, GQ_ERR_NONFINITE, GQ_ERR_NO_CALIBRATION, GQ_ERR_HIP, GQ_ERR_INTERNAL,
 GQ_ERR_IO) = range(8)
GQ_HFQM_F32, GQ_HFQM_HESSIAN = 0, 130
GQ_STATIC_GROUPS, GQ_NF4, GQ_ACT_ORDER = 1, 2, 4
GQ_F32, GQ_BF16 = 0, 1
GQ_PSD_AUTO, GQ_PSD_F64 = 0, 1
GQ_SWEEP_AUTO, GQ_SWEEP_F32, GQ_SWEEP_F64 = 0, 1, 2

EXPORTS = (
    "gq_abi_version", "gq_last_error", "hessian_accumulate", "hessian_tril_bytes",
    "hessian_pack_tril", "hessian_unpack_tril", "psd_project_workspace_size", "psd_project",
    "psd_project_flops", "psd_project_products", "gq_set_timing", "psd_project_last_timing", "gq_set_psd_products",
    "gq_set_sweep_state",
    "gptq_factor_workspace_size", "gptq_factor", "gptq_sweep_workspace_size", "gptq_sweep",
    "gptq_factor_f64", "gptq_sweep_f64_workspace_size", "gptq_sweep_f64",
    "gptq_quantize_workspace_size", "gptq_quantize", "rtn_quantize_workspace_size", "rtn_quantize",
    "gptq_sweep_ex", "gptq_quantize_ex", "rtn_quantize_ex", "gq_nf4_levels", "gptq_quantize_ex_workspace_size",
    "hfqm_write", "hfqm_read_header", "hfqm_read_entry", "hfqm_read_payload",
    "hadamard_rotate_rows", "hadamard_rotate_hessian_workspace_size", "hadamard_rotate_hessian",
    "rtn_quantize_noalloc", "hessian_accumulate_chunks_workspace_size", "hessian_accumulate_chunks",
)


class GQError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed with status {status}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m post_weight_quantization_accumulate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, SZ, F, D = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t,
                               ctypes.c_float, ctypes.c_double)
        U32 = ctypes.c_uint32
        sig = {
            "gq_abi_version": (I, []),
            "gq_last_error": (ctypes.c_char_p, []),
            "hessian_accumulate": (I, [P, P, I, I64, I64, P]),
            "hessian_tril_bytes": (SZ, [I64]),
            "hessian_accumulate_chunks_workspace_size": (SZ, [I64, I64]),
            "hessian_accumulate_chunks": (I, [P, P, P, I64, I, I64, P, SZ, P]),
            "hessian_pack_tril": (I, [P, P, I64, P]),
            "hessian_unpack_tril": (I, [P, P, I64, P]),
            "psd_project_workspace_size": (SZ, [I64]),
            "psd_project": (I, [P, I64, P, SZ, P]),
            "psd_project_flops": (D, [I64]),
            "psd_project_products": (I, []),
            "gq_set_timing": (None, [I]),
            "gq_set_psd_products": (I, [I]),
            "gq_set_sweep_state": (I, [I]),
            "psd_project_last_timing": (I, [ctypes.POINTER(I), ctypes.POINTER(D), ctypes.POINTER(ctypes.c_char_p)]),
            "gptq_factor_workspace_size": (SZ, [I64]),
            "gptq_factor": (I, [P, P, I64, F, P, SZ, P]),
            "gptq_sweep_workspace_size": (SZ, [I64, I64, I64]),
            "gptq_sweep": (I, [P, P, P, P, P, P, I64, I64, I64, P, SZ, P]),
            "gptq_factor_f64": (I, [P, P, I64, F, P, SZ, P]),
            "gptq_sweep_f64_workspace_size": (SZ, [I64, I64, I64]),
            "gptq_sweep_f64": (I, [P, P, P, P, P, P, I64, I64, I64, P, SZ, P]),
            "gptq_quantize_workspace_size": (SZ, [I64, I64, I64]),
            "gptq_quantize": (I, [P, P, P, P, P, P, I64, I64, I64, F, P, SZ, P]),
            "rtn_quantize_workspace_size": (SZ, [I64, I64, I64]),
            "rtn_quantize": (I, [P, P, P, P, P, I64, I64, I64, P, SZ, P]),
            "rtn_quantize_ex": (I, [P, P, P, P, P, I64, I64, I64, U32, P, SZ, P]),
            "rtn_quantize_noalloc": (I, [P, P, P, P, P, I64, I64, I64, U32, P]),
            "gptq_sweep_ex": (I, [P, P, P, P, P, P, I64, I64, I64, U32, P, SZ, P]),
            "gptq_quantize_ex": (I, [P, P, P, P, P, P, I64, I64, I64, F, U32, P, SZ, P]),
            "gq_nf4_levels": (None, [P]),
            "gptq_quantize_ex_workspace_size": (SZ, [I64, I64, I64, U32]),
            "hfqm_write": (I, [ctypes.c_char_p, ctypes.c_uint32, ctypes.c_char_p, I64, P, P, P, P, P, P, P]),
            "hfqm_read_header": (I, [ctypes.c_char_p, P, P, P, P, SZ, P]),
            "hfqm_read_entry": (I, [ctypes.c_char_p, I64, P, SZ, P, P, P, P, P, P]),
            "hfqm_read_payload": (I, [ctypes.c_char_p, I64, P, SZ]),
            "hadamard_rotate_rows": (I, [P, I64, I64, I64, I64, P, P]),
            "hadamard_rotate_hessian_workspace_size": (SZ, [I64]),
            "hadamard_rotate_hessian": (I, [P, I64, I64, P, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, numel=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _check(status: int, what: str):
    if status != GQ_OK:
        raise GQError(status, what, lib().gq_last_error().decode(errors="replace"))


def abi_version() -> int:
    return lib().gq_abi_version()


def workspace(nbytes: int, device) -> torch.Tensor:
    """A byte buffer to pass as `ws` (the library itself never allocates)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def hessian_accumulate(H: torch.Tensor, X: torch.Tensor) -> None:
    """H[i][j] += sum_t X[t][i] X[t][j] for i >= j (fp32 H, fp32 or bf16 X)."""
    T, K = X.shape
    _need(H, "H", torch.float32, K * K)
    _need(X, "X", None)
    if X.dtype == torch.bfloat16:
        dt = GQ_BF16
    elif X.dtype == torch.float32:
        dt = GQ_F32
    else:
        raise ValueError("X must be fp32 or bf16")
    _check(lib().hessian_accumulate(_ptr(H), _ptr(X), dt, T, K, _stream(H)), "hessian_accumulate")


def hessian_accumulate_chunks_workspace_size(K: int, n: int) -> int:
    return int(lib().hessian_accumulate_chunks_workspace_size(K, n))


def hessian_accumulate_chunks(H: torch.Tensor, chunks, ws=None) -> None:
    """H[i][j] += sum over the chunks of sum_t X[t][i] X[t][j] for i >= j, in as
    few launches as the library can (all chunks fp32 or all bf16, same K)."""
    n = len(chunks)
    if n == 0:
        return
    K = chunks[0].shape[1]
    _need(H, "H", torch.float32, K * K)
    dtypes = {X.dtype for X in chunks}
    if len(dtypes) != 1 or next(iter(dtypes)) not in (torch.float32, torch.bfloat16):
        raise ValueError("chunks must be all fp32 or all bf16")
    for X in chunks:
        _need(X, "X", None)
        if X.shape[1] != K:
            raise ValueError("every chunk needs K columns")
    dt = GQ_BF16 if chunks[0].dtype == torch.bfloat16 else GQ_F32
    ptrs = (ctypes.c_void_p * n)(*[X.data_ptr() for X in chunks])
    toks = (ctypes.c_int64 * n)(*[X.shape[0] for X in chunks])
    if ws is not None:
        _need(ws, "ws", torch.uint8)
    _check(lib().hessian_accumulate_chunks(_ptr(H), ptrs, toks, n, dt, K, _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(H)), "hessian_accumulate_chunks")


def hessian_tril_bytes(K: int) -> int:
    return int(lib().hessian_tril_bytes(K))


def hessian_pack_tril(blob: torch.Tensor, H: torch.Tensor) -> None:
    K = H.shape[0]
    _need(H, "H", torch.float32, K * K)
    _need(blob, "blob", torch.uint8, hessian_tril_bytes(K))
    _check(lib().hessian_pack_tril(_ptr(blob), _ptr(H), K, _stream(H)), "hessian_pack_tril")


def hessian_unpack_tril(H: torch.Tensor, blob: torch.Tensor) -> None:
    K = H.shape[0]
    _need(H, "H", torch.float32, K * K)
    _need(blob, "blob", torch.uint8, hessian_tril_bytes(K))
    _check(lib().hessian_unpack_tril(_ptr(H), _ptr(blob), K, _stream(H)), "hessian_unpack_tril")


def psd_project_workspace_size(K: int) -> int:
    return int(lib().psd_project_workspace_size(K))


def psd_project_flops(K: int) -> float:
    return float(lib().psd_project_flops(K))


def psd_project_products() -> int:
    return int(lib().psd_project_products())


def gq_set_timing(on: bool) -> None:
    """Per-kernel event timing of later psd_project calls on this thread."""
    lib().gq_set_timing(1 if on else 0)


def gq_set_psd_products(kind: int) -> None:
    """GQ_PSD_AUTO or GQ_PSD_F64: kind of the products of later psd_project calls
    on this thread."""
    _check(lib().gq_set_psd_products(int(kind)), "gq_set_psd_products")


def gq_set_sweep_state(kind: int) -> None:
    """GQ_SWEEP_AUTO, GQ_SWEEP_F32 or GQ_SWEEP_F64: state of gptq_quantize's plain
    sweep in later calls on this thread."""
    _check(lib().gq_set_sweep_state(int(kind)), "gq_set_sweep_state")


def psd_project_last_timing():
    """(launches, summed ms, kernel name) of the product kernel in the last timed
    psd_project call on this thread."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    name = ctypes.c_char_p()
    _check(lib().psd_project_last_timing(ctypes.byref(n), ctypes.byref(ms), ctypes.byref(name)),
           "psd_project_last_timing")
    return n.value, ms.value, name.value.decode()


def psd_project(H: torch.Tensor, ws: torch.Tensor) -> None:
    K = H.shape[0]
    _need(H, "H", torch.float32, K * K)
    _need(ws, "ws", torch.uint8)
    _check(lib().psd_project(_ptr(H), K, _ptr(ws), ws.numel(), _stream(H)), "psd_project")


def gptq_factor_workspace_size(K: int) -> int:
    return int(lib().gptq_factor_workspace_size(K))


def gptq_factor(U: torch.Tensor, H: torch.Tensor, damp: float, ws: torch.Tensor) -> None:
    K = H.shape[0]
    _need(U, "U", torch.float32, K * K)
    _need(H, "H", torch.float32, K * K)
    _need(ws, "ws", torch.uint8)
    _check(lib().gptq_factor(_ptr(U), _ptr(H), K, float(damp), _ptr(ws), ws.numel(), _stream(H)),
           "gptq_factor")


def gptq_sweep_workspace_size(N: int, K: int, group: int) -> int:
    return int(lib().gptq_sweep_workspace_size(N, K, group))


def _quant_args(codes, scales, W, M, imp, group, ws, mname):
    N, K = W.shape
    _need(W, "W", torch.float32)
    if M is not None:
        _need(M, mname, torch.float32, K * K)
    _need(codes, "codes", torch.uint8, N * (K // 2))
    _need(scales, "scales", torch.float32, N * (K // max(group, 1)))
    if imp is not None:
        _need(imp, "imp", torch.float32, K)
    _need(ws, "ws", torch.uint8)
    return N, K


def gptq_sweep(codes, scales, W, U, imp, group: int, ws, want_qerr: bool = True):
    """Codes/scales of the GPTQ sweep of W under U; returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, U, imp, group, ws, "U")
    q = ctypes.c_double(0.0)
    _check(lib().gptq_sweep(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                            _ptr(W), _ptr(U), _ptr(imp), N, K, group, _ptr(ws), ws.numel(),
                            _stream(W)), "gptq_sweep")
    return q.value if want_qerr else None


def gptq_factor_f64(U: torch.Tensor, H: torch.Tensor, damp: float, ws: torch.Tensor) -> None:
    """gptq_factor with U (K x K float64) kept in fp64."""
    K = H.shape[0]
    _need(U, "U", torch.float64, K * K)
    _need(H, "H", torch.float32, K * K)
    _need(ws, "ws", torch.uint8)
    _check(lib().gptq_factor_f64(_ptr(U), _ptr(H), K, float(damp), _ptr(ws), ws.numel(), _stream(H)),
           "gptq_factor_f64")


def gptq_sweep_f64_workspace_size(N: int, K: int, group: int) -> int:
    return int(lib().gptq_sweep_f64_workspace_size(N, K, group))


def gptq_sweep_f64(codes, scales, W, U, imp, group: int, ws, want_qerr: bool = True):
    """gptq_sweep with its state in fp64 under a float64 U from gptq_factor_f64;
    returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, None, imp, group, ws, "U")
    _need(U, "U", torch.float64, K * K)
    q = ctypes.c_double(0.0)
    _check(lib().gptq_sweep_f64(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                                _ptr(W), _ptr(U), _ptr(imp), N, K, group, _ptr(ws), ws.numel(),
                                _stream(W)), "gptq_sweep_f64")
    return q.value if want_qerr else None


def gptq_sweep_ex(codes, scales, W, U, imp, group: int, flags: int, ws, want_qerr: bool = True):
    """gptq_sweep with flags (GQ_STATIC_GROUPS, GQ_NF4); returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, U, imp, group, ws, "U")
    q = ctypes.c_double(0.0)
    _check(lib().gptq_sweep_ex(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                               _ptr(W), _ptr(U), _ptr(imp), N, K, group, flags, _ptr(ws), ws.numel(),
                               _stream(W)), "gptq_sweep_ex")
    return q.value if want_qerr else None


def nf4_levels():
    """The library's 16 NF4 levels (fp32, ascending) as a host tensor."""
    out = (ctypes.c_float * 16)()
    lib().gq_nf4_levels(out)
    return torch.tensor(list(out), dtype=torch.float32)


def rtn_quantize_workspace_size(N: int, K: int, group: int) -> int:
    return int(lib().rtn_quantize_workspace_size(N, K, group))


def rtn_quantize(codes, scales, W, imp, group: int, ws, want_qerr: bool = True):
    """Round-to-nearest codes/scales of W on the sweep's grid; returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, None, imp, group, ws, "")
    q = ctypes.c_double(0.0)
    _check(lib().rtn_quantize(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                              _ptr(W), _ptr(imp), N, K, group, _ptr(ws), ws.numel(), _stream(W)), "rtn_quantize")
    return q.value if want_qerr else None


def rtn_quantize_ex(codes, scales, W, imp, group: int, flags: int, ws, want_qerr: bool = True):
    """rtn_quantize with flags (GQ_NF4); returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, None, imp, group, ws, "")
    q = ctypes.c_double(0.0)
    _check(lib().rtn_quantize_ex(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                                 _ptr(W), _ptr(imp), N, K, group, flags, _ptr(ws), ws.numel(), _stream(W)),
           "rtn_quantize_ex")
    return q.value if want_qerr else None


NOALLOC_SCRATCH_BYTES = 65536      # GQ_NOALLOC_SCRATCH_BYTES of include/gq.h


def rtn_quantize_noalloc(codes, scales, W, imp, group: int, flags: int = 0, want_qerr: bool = True):
    """rtn_quantize_ex without a workspace (the library's fixed per-device
    scratch; calls that overlap on one device race); returns qerr (or None)."""
    N, K = W.shape
    _need(W, "W", torch.float32)
    _need(codes, "codes", torch.uint8, N * (K // 2))
    _need(scales, "scales", torch.float32, N * (K // max(group, 1)))
    if imp is not None:
        _need(imp, "imp", torch.float32, K)
    q = ctypes.c_double(0.0)
    _check(lib().rtn_quantize_noalloc(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                                      _ptr(W), _ptr(imp), N, K, group, flags, _stream(W)),
           "rtn_quantize_noalloc")
    return q.value if want_qerr else None


def gptq_quantize_workspace_size(N: int, K: int, group: int) -> int:
    return int(lib().gptq_quantize_workspace_size(N, K, group))


def gptq_quantize_ex_workspace_size(N: int, K: int, group: int, flags: int) -> int:
    return int(lib().gptq_quantize_ex_workspace_size(N, K, group, flags))


def gptq_quantize_ex(codes, scales, W, H, imp, group: int, damp: float, flags: int, ws, want_qerr: bool = True):
    """gptq_quantize with flags (GQ_STATIC_GROUPS, GQ_NF4, GQ_ACT_ORDER); returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, H, imp, group, ws, "H")
    q = ctypes.c_double(0.0)
    _check(lib().gptq_quantize_ex(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                                  _ptr(W), _ptr(H), _ptr(imp), N, K, group, float(damp), flags, _ptr(ws),
                                  ws.numel(), _stream(W)), "gptq_quantize_ex")
    return q.value if want_qerr else None


def gptq_quantize(codes, scales, W, H, imp, group: int, damp: float, ws, want_qerr: bool = True):
    """Damping, Cholesky, U and the sweep in one call; returns qerr (or None)."""
    N, K = _quant_args(codes, scales, W, H, imp, group, ws, "H")
    q = ctypes.c_double(0.0)
    _check(lib().gptq_quantize(_ptr(codes), _ptr(scales), ctypes.byref(q) if want_qerr else None,
                               _ptr(W), _ptr(H), _ptr(imp), N, K, group, float(damp), _ptr(ws),
                               ws.numel(), _stream(W)), "gptq_quantize")
    return q.value if want_qerr else None


# ------------------------------------------------------------------ Hadamard rotation
def hadamard_rotate_rows(A, block: int, signs=None):
    """A[r, :] <- A[r, :] R^T in place for an fp32 (rows x K) tensor (row stride may exceed K)."""
    if not isinstance(A, torch.Tensor) or not A.is_cuda or A.dtype != torch.float32:
        raise ValueError("A must be a CUDA (HIP) float32 tensor")
    if A.dim() != 2 or A.stride(1) != 1:
        raise ValueError("A must be 2-D with unit column stride")
    rows, K = A.shape
    if signs is not None:
        _need(signs, "signs", torch.float32, K)
    _check(lib().hadamard_rotate_rows(_ptr(A), rows, K, A.stride(0), block, _ptr(signs), _stream(A)),
           "hadamard_rotate_rows")


def hadamard_rotate_hessian_workspace_size(K: int) -> int:
    return int(lib().hadamard_rotate_hessian_workspace_size(K))


def hadamard_rotate_hessian(H, block: int, ws, signs=None):
    """H <- R H R^T in place for a full symmetric fp32 K x K tensor."""
    K = H.shape[0]
    _need(H, "H", torch.float32, K * K)
    _need(ws, "ws", torch.uint8)
    if signs is not None:
        _need(signs, "signs", torch.float32, K)
    _check(lib().hadamard_rotate_hessian(_ptr(H), K, block, _ptr(signs), _ptr(ws), ws.numel(), _stream(H)),
           "hadamard_rotate_hessian")


# ------------------------------------------------------------------ HFQM package
def _host_bytes(x) -> "np.ndarray":
    import numpy as np
    if isinstance(x, torch.Tensor):
        x = x.detach().contiguous().view(torch.uint8).cpu().numpy()
    return np.ascontiguousarray(np.frombuffer(memoryview(x).cast("B"), dtype=np.uint8))


def hfqm_write(path: str, arch_id: int, metadata: str, entries):
    """Write an HFQM package.  entries: (name, quant_type, shape, group_size, payload)
    in index order; payload is bytes, a numpy array or a tensor (host or device)."""
    n = len(entries)
    names = (ctypes.c_char_p * max(n, 1))(*[e[0].encode() for e in entries])
    qts = (ctypes.c_uint8 * max(n, 1))(*[e[1] for e in entries])
    nds = (ctypes.c_uint8 * max(n, 1))(*[len(e[2]) for e in entries])
    shp = (ctypes.c_uint32 * max(4 * n, 1))()
    for i, e in enumerate(entries):
        if len(e[2]) > 4:
            raise ValueError("at most 4 dimensions per entry")
        for d, v in enumerate(e[2]):
            shp[4 * i + d] = v
    grp = (ctypes.c_uint32 * max(n, 1))(*[e[3] for e in entries])
    bufs = [_host_bytes(e[4]) for e in entries]
    sizes = (ctypes.c_uint64 * max(n, 1))(*[b.size for b in bufs])
    data = (ctypes.c_void_p * max(n, 1))(*[b.ctypes.data for b in bufs])
    _check(lib().hfqm_write(path.encode(), arch_id, metadata.encode(), n, names, qts, nds, shp, grp, sizes, data),
           "hfqm_write")


def hfqm_read(path: str):
    """(arch_id, metadata JSON text, [(name, quant_type, shape, group_size, data_size, offset)])."""
    arch, n, doff, mlen = ctypes.c_uint32(), ctypes.c_int64(), ctypes.c_uint64(), ctypes.c_size_t()
    _check(lib().hfqm_read_header(path.encode(), ctypes.byref(arch), ctypes.byref(n), ctypes.byref(doff), None, 0,
                                  ctypes.byref(mlen)), "hfqm_read_header")
    meta = ctypes.create_string_buffer(mlen.value + 1)
    _check(lib().hfqm_read_header(path.encode(), None, None, None, meta, mlen.value + 1, None), "hfqm_read_header")
    out = []
    for i in range(n.value):
        name = ctypes.create_string_buffer(65536)
        qt, nd = ctypes.c_uint8(), ctypes.c_uint8()
        shape = (ctypes.c_uint32 * 4)()
        grp, size, off = ctypes.c_uint32(), ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().hfqm_read_entry(path.encode(), i, name, 65536, ctypes.byref(qt), ctypes.byref(nd), shape,
                                     ctypes.byref(grp), ctypes.byref(size), ctypes.byref(off)), "hfqm_read_entry")
        out.append((name.value.decode(), qt.value, tuple(shape[:nd.value]), grp.value, size.value, off.value))
    return arch.value, meta.value.decode(), out


def hfqm_read_payload(path: str, i: int, size: int):
    """Entry i's payload (size bytes, from hfqm_read) as a numpy uint8 array."""
    import numpy as np
    dst = np.empty(size, np.uint8)
    _check(lib().hfqm_read_payload(path.encode(), i, dst.ctypes.data if size else None, size), "hfqm_read_payload")
    return dst

