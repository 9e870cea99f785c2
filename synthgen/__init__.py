"""Seeded, counter-based synthetic inputs for the calibration-Hessian GPTQ path.

This module is shared by the tests, the benchmark and the CPU reference: it only
makes inputs (activations X, weights W) and holds none of the method's
arithmetic (no Gram, no storage format, no factorisation, no quantisation).

Every value is a pure function of (seed, stream, global index):

    key  = (seed << 48) ^ (stream << 40) ^ index          (index < 2**40)
    h    = SplitMix64 output number `key`                   i.e. mix((key + 1) * gamma)
    u    = (h >> 11) * 2**-53                               uniform on [0, 1)
    N(0,1) by Box-Muller on index pairs (2p, 2p+1) of the uniform stream,
    cos for even element indices, sin for odd ones, in float64.

SplitMix64 is Steele, Lea & Flood (OOPSLA 2014), "Fast splittable pseudorandom
number generators"; gamma = 0x9E3779B97F4A7C15 and the two mixing multipliers are
the published ones.  Because every element is addressable on its own, chunks of a
stream (token ranges, row ranges) reproduce exactly, whatever device or chunking
generates them.

The workloads mirror the shapes the pages discuss: K=5120 is the attention
projection size the dataset card measures (hipfire-calib-data, "REQUIRED: project
to PSD before Cholesky"), K=17408 the size at which stored Hessians always fail
Cholesky (same section, table of K against lambda_min), and the streamed case
is a scaled-down calibration run whose statistic is a sum over chunks
(AtomicChat Qwen3.8-27B GGUF page, "The importance matrix").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# ---------------------------------------------------------------- generator core
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(u: int) -> int:
    """Unsigned 64-bit constant as the signed int64 torch stores."""
    return u - (1 << 64) if u >= (1 << 63) else u


_GAMMA_S, _M1_S, _M2_S = _s64(_GAMMA), _s64(_M1), _s64(_M2)

# stream ids
S_X, S_W, S_A, S_F, S_E, S_S, S_O, S_Z, S_L, S_T1, S_T2, S_T3 = range(1, 13)
S_W_BASE = 32  # S_W_BASE + t for the t-th weight tensor of a multi-tensor workload


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def splitmix64_mix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output mixing of int64 bit patterns (wrapping arithmetic)."""
    z = (z ^ _srl(z, 30)) * _M1_S
    z = (z ^ _srl(z, 27)) * _M2_S
    return z ^ _srl(z, 31)


def hash64(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output number key(seed, stream, index), as int64 bit patterns."""
    key = index ^ ((seed << 48) | (stream << 40))
    return splitmix64_mix((key + 1) * _GAMMA_S)


def uniform(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """float64 uniform on [0, 1) with 53 random bits."""
    return _srl(hash64(seed, stream, index), 11).to(torch.float64) * (2.0 ** -53)


def normal(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """float64 standard normal for each element index (Box-Muller on index pairs)."""
    p = index >> 1
    u1 = uniform(seed, stream, 2 * p)
    u2 = uniform(seed, stream, 2 * p + 1)
    r = torch.sqrt(-2.0 * torch.log1p(-u1))
    th = (2.0 * math.pi) * u2
    return torch.where((index & 1) == 0, r * torch.cos(th), r * torch.sin(th))


_CHUNK = 1 << 23


def _fill(fn, seed, stream, shape, offset=0, device="cpu"):
    """Evaluate fn(seed, stream, flat_index) over a row-major tensor of `shape`."""
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=torch.float64, device=device)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        idx = torch.arange(a + offset, b + offset, dtype=torch.int64, device=device)
        out[a:b] = fn(seed, stream, idx)
    return out.view(*shape)


def normal_tensor(seed, stream, shape, offset=0, device="cpu"):
    return _fill(normal, seed, stream, shape, offset, device)


def uniform_tensor(seed, stream, shape, offset=0, device="cpu"):
    return _fill(uniform, seed, stream, shape, offset, device)


def to_bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 with round-to-nearest-even (torch's conversion)."""
    return x.to(torch.float32).to(torch.bfloat16)


# ---------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    T: int            # tokens per accumulation call
    K: int            # input channels (Hessian size)
    N: list           # output rows of each weight tensor
    group: int
    damp: float
    x_dtype: str      # "f32" or "bf16"
    stored: bool      # Hessian goes through the bf16 tril storage + PSD projection
    chunks: int = 1   # accumulation calls
    seed: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 512, 128, [64], 32, 0.01, "f32", False, 1, 0),
    "stored1024": Workload("stored1024", 4096, 1024, [1024], 128, 0.01, "f32", True, 1, 1),
    "attn5120": Workload("attn5120", 8192, 5120, [10240], 128, 0.01, "bf16", True, 1, 2),
    "mlpdown17408": Workload("mlpdown17408", 8192, 17408, [5120], 128, 0.01, "bf16", True, 1, 3),
    "stream5120": Workload("stream5120", 8192, 5120, [5120, 10240, 1024, 1024], 128, 0.01,
                           "bf16", True, 128, 4),
}


def x_chunk(wl: Workload, chunk: int = 0, device="cpu", tokens=None) -> torch.Tensor:
    """Activation chunk `chunk` of workload `wl` (T x K row-major, fp32 or bf16).

    `tokens` restricts the chunk to its first `tokens` rows (used for small tests
    with the same recipe).
    """
    T = wl.T if tokens is None else tokens
    K, seed = wl.K, wl.seed
    if wl.name == "tiny":
        return normal_tensor(seed, S_X, (T, K), device=device).to(torch.float32)
    if wl.name == "stored1024":
        # X = Z . L, L lower triangular: L_ii = exp(-4 i / K), L_ij ~ N(0, 1/K) for i > j
        Z = normal_tensor(seed, S_Z, (T, K), device=device)
        L = normal_tensor(seed, S_L, (K, K), device=device) / math.sqrt(K)
        L = torch.tril(L, diagonal=-1)
        L = L + torch.diag(torch.exp(-4.0 * torch.arange(K, dtype=torch.float64, device=device) / K))
        return (Z @ L).to(torch.float32)
    if wl.name in ("attn5120", "stream5120"):
        rank = 256 if wl.name == "attn5120" else 512
        total_tokens = wl.T * wl.chunks
        c = 1.0 / math.sqrt(total_tokens * 1.01)
        A = normal_tensor(seed, S_A, (rank, K), device=device) / math.sqrt(rank)
        row0 = chunk * wl.T
        F = normal_tensor(seed, S_F, (T, rank), offset=row0 * rank, device=device)
        E = normal_tensor(seed, S_E, (T, K), offset=row0 * K, device=device)
        X = c * (F @ A + 0.1 * E)
        return to_bf16_rne(X.to(torch.float32))
    if wl.name == "mlpdown17408":
        return heavy_tailed_x(seed, T, K, wl.T, device=device)
    raise KeyError(wl.name)


def heavy_tailed_x(seed: int, T: int, K: int, T_norm: int, device="cpu") -> torch.Tensor:
    """Student-t (nu = 3) activations with log-normal (sigma = 1) per-channel
    scales, as bf16: t = z / sqrt(chi2_3 / 3), x = c s_k t with s_k = exp(N(0,1))
    and c = 1 / sqrt(T_norm * 3 * mean(s^2)), so that mean(diag X^T X) is about 1
    over T_norm tokens.  The MLP down-projection recipe (K = 17408) and its
    smaller blocks."""
    z = normal_tensor(seed, S_X, (T, K), device=device)
    chi2 = (normal_tensor(seed, S_T1, (T, K), device=device) ** 2
            + normal_tensor(seed, S_T2, (T, K), device=device) ** 2
            + normal_tensor(seed, S_T3, (T, K), device=device) ** 2)
    t = z / torch.sqrt(chi2 / 3.0)
    del z, chi2
    s = torch.exp(normal_tensor(seed, S_S, (K,), device=device))
    c = 1.0 / math.sqrt(T_norm * 3.0 * float((s * s).mean()))
    return to_bf16_rne((c * s[None, :] * t).to(torch.float32))


def common_mode_x(seed: int, T: int, K: int, device="cpu") -> torch.Tensor:
    """Strongly correlated activations, as bf16: one factor shared by every
    channel, x_tk = c (0.88 u_t m_k + 0.45 z_tk) with u, z ~ N(0, 1) and loadings
    m_k = 1 + 0.05 N(0, 1), c = 1 / sqrt(T (0.88^2 + 0.45^2)).  Their Gram matrix
    has a mean diagonal near 1 and off-diagonal entries near 0.77, like the
    dataset card's K=5120 tensor (mean diag 0.995, off-diagonal RMS 0.789), so
    the truncated storage of it leaves sizeable negative eigenvalues when
    T < K."""
    u = normal_tensor(seed, S_F, (T, 1), device=device)
    m = 1.0 + 0.05 * normal_tensor(seed, S_A, (1, K), device=device)
    z = normal_tensor(seed, S_E, (T, K), device=device)
    c = 1.0 / math.sqrt(T * (0.88 ** 2 + 0.45 ** 2))
    return to_bf16_rne((c * (0.88 * u * m + 0.45 * z)).to(torch.float32))


def weights(wl: Workload, t: int = 0, device="cpu", rows=None) -> torch.Tensor:
    """Weight tensor t of workload `wl` (N x K fp32 row-major); `rows` limits N."""
    N = wl.N[t] if rows is None else rows
    K, seed = wl.K, wl.seed
    if wl.name == "tiny":
        return (2.0 * uniform_tensor(seed, S_W, (N, K), device=device) - 1.0).to(torch.float32)
    if wl.name == "stored1024":
        return (0.02 * normal_tensor(seed, S_W, (N, K), device=device)).to(torch.float32)
    if wl.name == "attn5120":
        w = 0.02 * normal_tensor(seed, S_W, (N, K), device=device)
        o = uniform_tensor(seed, S_O, (N, K), device=device) < 0.001
        return torch.where(o, 20.0 * w, w).to(torch.float32)
    if wl.name == "mlpdown17408":
        return (0.015 * normal_tensor(seed, S_W, (N, K), device=device)).to(torch.float32)
    if wl.name == "stream5120":
        return (0.02 * normal_tensor(seed, S_W_BASE + t, (N, K), device=device)).to(torch.float32)
    raise KeyError(wl.name)


def uniform_weights(seed: int, N: int, K: int, device="cpu") -> torch.Tensor:
    """W ~ U(-1, 1), the distribution the ork-driver qerr check uses."""
    return (2.0 * uniform_tensor(seed, S_W, (N, K), device=device) - 1.0).to(torch.float32)


def normal_matrix(seed: int, stream: int, rows: int, cols: int, scale: float = 1.0,
                  device="cpu") -> torch.Tensor:
    """Plain N(0, scale^2) fp32 matrix from stream `stream` (test helper)."""
    return (scale * normal_tensor(seed, stream, (rows, cols), device=device)).to(torch.float32)
