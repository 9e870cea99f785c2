// gq_internal.h -- shared declarations of the HIP implementation (gfx950).
//
// Device status word bits, the TN matrix-core GEMM interface used by every dense
// contraction of the path (Gram in fp32, Cholesky/inverse and the sign iteration
// in fp64, GPTQ lazy-block update in fp32), and the launchers of the other
// kernels.  Host code in api.hip orchestrates them.
#pragma once

#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>
#include <stddef.h>

namespace gq {

// Calls f(std::integral_constant<int, I>{}) for I = 0, 1, ..., N-1: a loop whose
// index is a compile-time constant in the body.
template <typename F, int... I> __device__ inline void static_for_impl(F &f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ inline void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Bits of the device status word (OR-ed by kernels, read once per call).
enum : unsigned {
    ST_NOT_PD = 1u,      // a Cholesky pivot was not > 0
    ST_NONFINITE = 2u,   // NaN / Inf in an input
    ST_NO_CALIB = 4u,    // mean(diag H) <= 0 (or not finite)
    ST_RANGE = 8u,       // an emulated product's output left the range its split form needs
};

// Tile order of the large-tile kernels.  Workgroups are dispatched round-robin
// over the chip's 8 XCDs (workgroup w runs on XCD w % 8, each with its own L2):
// xcd_order gives each XCD a contiguous range of logical tile indices, and
// lower_tile_grouped walks the lower triangle (ti >= tj) of an nt x nt grid in
// groups of kTileGroup tile rows, so tiles that run together on one XCD share
// their row and column panels in its L2.
constexpr int kXcds = 8;
constexpr int64_t kTileGroup = 4;

__device__ inline int64_t xcd_order(int64_t w, int64_t n)
{
    const int64_t x = w % kXcds, j = w / kXcds;
    int64_t base = 0;
    for (int64_t y = 0; y < x; ++y) base += (n - y + kXcds - 1) / kXcds;
    return base + j;
}

__device__ inline void lower_tile_grouped(int64_t l, int64_t nt, int64_t &ti, int64_t &tj)
{
    int64_t g = 0, start = 0;
    for (;;) {
        const int64_t r0 = g * kTileGroup;
        const int64_t r1 = (r0 + kTileGroup < nt) ? r0 + kTileGroup : nt;
        const int64_t cnt = (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2;
        if (l < start + cnt) {
            int64_t off = l - start;
            const int64_t full = r0 * (r1 - r0);
            if (off < full) {
                tj = off / (r1 - r0);
                ti = r0 + off % (r1 - r0);
            } else {
                off -= full;
                int64_t cc = r0;
                while (off >= r1 - cc) { off -= r1 - cc; ++cc; }
                tj = cc;
                ti = cc + off;
            }
            return;
        }
        start += cnt;
        ++g;
    }
}

// Which output tiles a GEMM launch computes.
enum TileMode : int { TILE_RECT = 0, TILE_LOWER = 1, TILE_UPPER = 2 };

// C(i, j) for i < M, j < N of
//     out = alpha * sum_{k < Kd} A[k*lda + i] * B[k*ldb + j] + beta * cin[i*ldc + j]
// Both operands are "k-major": row k of A holds the i-range, row k of B the
// j-range (the transposed-A, normal-B product A^T B).  alpha and beta are the
// host values times (*alpha_dev)^alpha_pow (resp. beta) when the device pointer
// is set.  tri = 1 keeps only i >= j, tri = 2 only i <= j.  When out_t is set,
// each kept (i, j) is also written at out_t[j*ldo + i] (the mirror; out_t is the
// origin of the transposed block, which for a symmetric output is out itself).
struct GemmDesc {
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    int64_t M, N, Kd;
    void *out; int64_t ldo;
    void *out_t;              // mirror base (may equal out), or nullptr
    const void *cin; int64_t ldc;   // same element type as A/B; may alias out
    double alpha, beta;
    const double *alpha_dev; int alpha_pow;
    const double *beta_dev; int beta_pow;
    int tri;
    int mode;                 // TileMode
};

// T = float or double; OutT = T, or float for a double product written as fp32.
hipError_t gemm_tn_f32(const GemmDesc &d, hipStream_t s);
hipError_t gemm_tn_f64(const GemmDesc &d, hipStream_t s);
hipError_t gemm_tn_f64_out_f32(const GemmDesc &d, hipStream_t s);
// Stream-K variants for products with at least as many tiles as resident
// workgroups (at most kStreamKMaxWorkers of them); with fewer tiles, or with no
// partials buffer, they run one tile per workgroup.  partials holds
// streamk_partials_bytes(sizeof element) bytes of scratch and flags
// kStreamKMaxWorkers counters, which must be zero before the first call and
// are left zero by every call.  out must not alias A, B or cin.
constexpr int64_t kStreamKMaxWorkers = 512;
constexpr size_t streamk_partials_bytes(size_t elem) { return (size_t)2 * kStreamKMaxWorkers * 128 * 128 * elem; }
// True when a lower-triangle product of order K has enough tiles for stream-K.
constexpr bool streamk_lower_worthwhile(int64_t K)
{
    return ((K + 127) / 128) * ((K + 127) / 128 + 1) / 2 >= kStreamKMaxWorkers;
}
hipError_t gemm_tn_f64_streamk(const GemmDesc &d, void *partials, unsigned *flags, hipStream_t s);
hipError_t gemm_tn_f64_out_f32_streamk(const GemmDesc &d, void *partials, unsigned *flags, hipStream_t s);

// Products of symmetric fp64 matrices by modular integer emulation on the int8
// matrix cores (ozaki.hip).  The split form of a K x K symmetric matrix Z holds
// the residues, modulo each of oz_mods(K) moduli, of its row-scaled integer form
// rint(Z_ik 2^(beta - e_i)) (oz_planes_bytes(K) bytes: oz_mods(K) planes of
// Kp x Kp int8 in blocks of 256 rows x 64 k, zero padded), with e_i either per
// row (rowexp) or one exponent
// for every row (entries below 2^exp in magnitude).  oz_split writes it with
// per-row exponents.  oz_product computes
//     out = alpha * A B + beta * cin   over the lower triangle (+ mirror)
// from the split forms of A and B: d carries out, out_t, ldo, cin, ldc, alpha,
// beta and their device factors, with M = N = Kd = K; out may be null.  With
// o.planes set it also writes the split form of (that value + o.diag_shift on
// the diagonal) at the single exponent o.exp (its padding must already be
// zero), and ORs ST_RANGE into *status if an entry reaches 2^o.exp.  Cres is
// oz_planes_bytes(K) bytes of scratch; beta is oz_beta(K) for every operand.
// after_gemm, if set, is recorded on s right after the int8 product kernel.
// A product of order K uses the first oz_mods(K) of kOzMaxMods moduli: 12 up to
// K = kOzFewModsMaxK (operands of 40 bits), 13 above (43-44 bits).
constexpr int kOzMaxMods = 13;
constexpr int64_t kOzFewModsMaxK = 8192;
struct OzConst {
    int nm;                                            // moduli in use
    int m[kOzMaxMods];
    double inv_m[kOzMaxMods];
    unsigned long long M_lo, M_hi;                     // M = prod m_r
};
struct OzOperand {
    const int8_t *planes;
    const int *rowexp;          // per-row exponents, or null for `exp` on every row
    int exp;
};
struct OzOut {
    int8_t *planes;             // null: no split form written
    int exp;
    double diag_shift;
};
int oz_mods(int64_t K);
const OzConst &oz_const(int nm);
int oz_beta(int64_t K);
int64_t oz_padded(int64_t K);
size_t oz_planes_bytes(int64_t K);
// rowmax, if set, holds each row's largest magnitude (fp64 bits), which the
// split then does not recompute.
hipError_t oz_split(const double *Z, int64_t K, int beta, int8_t *planes, int *rowexp, hipStream_t s,
                    const unsigned long long *rowmax = nullptr);
hipError_t oz_product(const GemmDesc &d, const OzOperand &A, const OzOperand &B, int beta, uint8_t *Cres,
                      bool out_f32, const OzOut &o, unsigned *status, hipStream_t s, hipEvent_t after_gemm = nullptr);
// Zeroes the padding of a split form that oz_product's CRT leaves unwritten
// (nothing when K is a multiple of 256).
hipError_t oz_clear_padding(int8_t *planes, int64_t K, hipStream_t s);

// bf16 Gram: H_lower += X^T X, X T x K bf16 row-major.
hipError_t launch_gram_bf16(float *H, const uint16_t *X, int64_t T, int64_t K, hipStream_t s);
// Up to kGramMaxChunks bf16 chunks (K % 8 == 0, 16-byte aligned) in one launch,
// passed by value; `splits` workgroups per tile each take a contiguous range of
// chunks, and with splits > 1 their tiles go through `part`
// (gram_split_bytes(K, splits) bytes) and are added to H in split order.
constexpr int kGramMaxChunks = 128;
struct GramChunks {
    const uint16_t *x[kGramMaxChunks];
    int64_t t[kGramMaxChunks];
    int n;
};
int64_t gram_tiles(int64_t K);
size_t gram_split_bytes(int64_t K, int splits);
hipError_t launch_gram_bf16_chunks(float *H, const GramChunks &ch, int64_t K, int splits, float *part,
                                   hipStream_t s);

// Bf16TrilDiagF32 storage.
hipError_t launch_tril_pack(uint8_t *blob, const float *H, int64_t K, hipStream_t s);
hipError_t launch_tril_unpack(float *H, const uint8_t *blob, int64_t K, hipStream_t s);

// Small helpers (factor.hip).
hipError_t launch_fill_f64(double *p, int64_t n, double v, hipStream_t s);
hipError_t launch_fill_u32(unsigned *p, int64_t n, unsigned v, hipStream_t s);
hipError_t launch_set_identity_f64(double *X, int64_t K, hipStream_t s);
// D = sym(lower(H)) in fp64; status |= NONFINITE on a non-finite lower entry.
// rowmax, if set (K entries, zeroed beforehand), receives each row's largest
// magnitude as the bits of an fp64.
hipError_t launch_sym_lower_to_f64(double *D, const float *H, int64_t K, unsigned *status,
                                   hipStream_t s, unsigned long long *rowmax = nullptr);
// out[0] = sqrt(sum of squares of a[0..n)), deterministic two-stage tree;
// partials holds kFrobParts doubles.
constexpr int64_t kFrobParts = 1024;
hipError_t launch_frobenius(double *out, const double *a, int64_t n, double *partials, hipStream_t s);
// out[0] = x[0]^px * y[0]^py (y optional), or 0 unless x[0] (and y[0]) are finite and > 0.
hipError_t launch_scalar_combine(double *out, const double *x, double px, const double *y, double py,
                                 hipStream_t s);
// mu[0] = mean(diag H); status |= NO_CALIB if !(mu > 0); NONFINITE if the lower
// triangle of H holds NaN/Inf.
hipError_t launch_diag_mean_check(double *mu, const float *H, int64_t K, unsigned *status,
                                  hipStream_t s);
// M[i][j] = H[K-1-i][K-1-j] (i <= j, fp64) + (i == j) * damp * mu[0].
hipError_t launch_damp_reverse(double *M, const float *H, int64_t K, double damp,
                               const double *mu, hipStream_t s);
// Cholesky / inverse panel width: the diagonal blocks are factored in one
// workgroup, and every trailing and inverse update is a GEMM of depth kPanel.
constexpr int kPanel = 128;
// Factor the nb x nb diagonal block at (p0, p0) of M (upper Cholesky, in place,
// mirrored below) and write 1 / R_kk to rinv (kPanel doubles, 1 past nb).
hipError_t launch_potrf_diag(double *M, int64_t K, int64_t p0, int nb, double *rinv, unsigned *status,
                             hipStream_t s);
// out = R^-T B for the factored nb x nb block R at (p0, p0) of M and its rinv:
// B is nb x ncols (ld ldb), out may equal B; with out_t set, the result is
// also written transposed (out_t[c * ldt + a]).
hipError_t launch_trsm_rt(const double *M, int64_t K, int64_t p0, int nb, const double *rinv, const double *B,
                          int64_t ldb, double *out, int64_t ldo, double *out_t, int64_t ldt, int64_t ncols,
                          hipStream_t s);
// U[i][j] = X[K-1-i][K-1-j] for i <= j (as fp32), 0 below the diagonal.
hipError_t launch_flip(float *U, const double *X, int64_t K, hipStream_t s);

// GPTQ (gptq.hip).
constexpr int kSweepBlock = 128;      // lazy-batch block width (columns)
// Two-level lazy batch: blocks are grouped kSweepSuper columns at a time.  A
// block's errors update the rest of its group at once; the columns beyond the
// group receive the whole group's errors in one product of depth kSweepSuper.
constexpr int kSweepSuper = 512;
hipError_t launch_copy_check(float *dst, const float *src, int64_t n, unsigned *status,
                             hipStream_t s);
hipError_t launch_check_finite(const float *x, int64_t n, unsigned *status, hipStream_t s);
// The NF4 codebook (QLoRA's 4-bit NormalFloat): 16 levels in [-1, 1], ascending,
// 0 at index 7; normal quantiles at evenly spaced probabilities, 7 below zero and
// 8 above, the outermost at 1 - (1/32 + 1/30)/2, scaled by the largest.  A value
// x = w / absmax takes the nearest level: the count of midpoints
// fl32(L[j] + L[j+1]) / 2 below x (a value on a midpoint takes the lower level).
constexpr float kNF4[16] = {
    -0x1p+0f,          -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
    -0x1.234496p-2f,   -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0.0f,
    0x1.45f602p-4f,    0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
    0x1.c3496ap-2f,    0x1.200f52p-1f,  0x1.722760p-1f,  0x1p+0f};
// Quantiser modes (bit set): scales fixed before the sweep from the original
// weights; the NF4 codebook (scale absmax, unsigned level index per nibble).
enum : int { MODE_STATIC = 1, MODE_NF4 = 2 };

// Sweep of one lazy block.  With MODE_STATIC the scales are read from `scales`
// (written beforehand for every row and group), not computed and stored.
// gidx (static groups only, else null): the group of each column of W's order,
// when the columns are not in their natural order (act order).
hipError_t launch_sweep_block(float *Wk, float *ET, uint8_t *codes, float *scales,
                              const float *U, int64_t N, int64_t K, int64_t G, int64_t b0, int mode,
                              const int *gidx, hipStream_t s);
// The sweep with its state in fp64 (sweep64.hip), plain int4 grid, dynamic
// groups: W64 = W (with the finite check); U64 = the flip of the factor's
// L^-1 (upper triangle, zeros below); one lazy block of the sweep at column b0
// over W64 (K x N errors of the block written k-major to ET, N apart).
hipError_t launch_w64(double *dst, const float *src, int64_t n, unsigned *status, hipStream_t s);
hipError_t launch_flip64(double *U, const double *X, int64_t K, hipStream_t s);
hipError_t launch_sweep64_block(double *Wk, double *ET, uint8_t *codes, float *scales, const double *U, int64_t N,
                                int64_t K, int64_t G, int64_t b0, hipStream_t s);
// Act order: perm[a] = the column with the a-th largest diagonal entry of H (ties
// in column order), inv its inverse, gidx[a] = perm[a] / G; Hp = H permuted on
// both sides (from H's lower triangle); Wk = W's columns permuted (with the finite
// check); codes put back in the original column order (packed nibbles).
hipError_t launch_act_perm(int *perm, int *inv, int *gidx, const float *H, int64_t K, int64_t G, hipStream_t s);
// tmp: K x K scratch for a full symmetric copy (or null: a direct gather).
hipError_t launch_perm_sym(float *Hp, const float *H, const int *perm, float *tmp, int64_t K, hipStream_t s);
hipError_t launch_gather_cols(float *Wk, const float *W, const int *perm, int64_t N, int64_t K, unsigned *status,
                              hipStream_t s);
hipError_t launch_unpermute_codes(uint8_t *codes, const uint8_t *cperm, const int *inv, int64_t N, int64_t K,
                                  hipStream_t s);
// Round-to-nearest codes and scales of W on the sweep's grid (gptq.hip): the
// uniform int4 grid, or NF4 with MODE_NF4 in mode.  With partials set, also
// qerr's partial sums (as launch_qerr's, *nparts pairs, at most
// rtn_partials(N, K)), ready for launch_qerr_reduce.
int64_t rtn_partials(int64_t N, int64_t K);
hipError_t launch_rtn(const float *W, uint8_t *codes, float *scales, const float *imp, double *partials, int64_t N,
                      int64_t K, int64_t G, int mode, unsigned *status, hipStream_t s, int64_t *nparts);
// qerr's partial sums: *nparts pairs (at most 1024 and at most rtn_partials(N, K))
// for launch_qerr_reduce.
hipError_t launch_qerr(double *partials, const float *W, const uint8_t *codes,
                       const float *scales, const float *imp, int64_t N, int64_t K, int64_t G, int mode,
                       hipStream_t s, int64_t *nparts);
hipError_t launch_qerr_reduce(double *out2, const double *partials, int64_t nparts,
                              hipStream_t s);
int64_t qerr_partials(int64_t N);

// Block Walsh-Hadamard rotation (hadamard.hip): A[r, :] <- A[r, :] R^T for rows
// r < rows (ld apart), R = blockdiag(H_b) diag(signs) / sqrt(b); signs may be
// null (all +1).  hadamard_block_ok: b a power of two <= 4096 dividing K.
bool hadamard_block_ok(int64_t K, int64_t b);
// With src set, the rows are read from src (same shape and stride) and the
// rotated rows written to A, for the vector kernel's cases only (b >= 16, K and
// ld multiples of 4, 16-byte aligned pointers; else hipErrorInvalidValue).
hipError_t launch_fwht_rows(float *A, int64_t rows, int64_t K, int64_t ld, int64_t b, const float *signs,
                            hipStream_t s, const float *src = nullptr);
// out = in^T for K x K row-major fp32 matrices (out and in distinct).
hipError_t launch_transpose(float *out, const float *in, int64_t K, hipStream_t s);

// Sets the message gq_last_error returns (defined in api.hip); returns status.
int set_error(int status, const char *msg);

}  // namespace gq
