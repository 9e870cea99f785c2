// api.hip -- the C ABI (include/gq.h): argument validation, workspace carving,
// launch order, and the single end-of-call read of the device status word.
// The library allocates nothing; every buffer comes from the caller.
#include <string>
#include <cmath>
#include <vector>
#include <algorithm>
#include <mutex>

#include "gq.h"
#include "gq_internal.h"

using namespace gq;

namespace {

thread_local std::string g_last_error;

// A second stream per (thread, device) on which gptq_factor runs each next
// diagonal block while the trailing update of the current panel runs on the
// caller's stream, and two events that order the two.  Created on first use at
// the default priority and kept until the process ends.
struct Lookahead {
    int dev = -1;
    hipStream_t side = nullptr;                        // trailing updates of the Cholesky
    hipStream_t inv = nullptr;                         // the triangular inverse, alongside
    hipEvent_t to_side = nullptr, to_main = nullptr, to_inv = nullptr, inv_done = nullptr;
};
thread_local std::vector<Lookahead> g_lookahead;

hipError_t lookahead_for_current_device(Lookahead **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    for (auto &l : g_lookahead)
        if (l.dev == dev) { *out = &l; return hipSuccess; }
    Lookahead l;
    l.dev = dev;
    if ((e = hipStreamCreateWithFlags(&l.side, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&l.inv, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&l.to_side, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&l.to_main, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&l.to_inv, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&l.inv_done, hipEventDisableTiming)) != hipSuccess) return e;
    g_lookahead.push_back(l);
    *out = &g_lookahead.back();
    return hipSuccess;
}

int fail(int status, const std::string &msg)
{
    g_last_error = msg;
    return status;
}

int hip_fail(hipError_t e, const char *where)
{
    return fail(GQ_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define GQ_HIP(call, where)                        \
    do {                                           \
        hipError_t e_ = (call);                    \
        if (e_ != hipSuccess) return hip_fail(e_, where); \
    } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves aligned sub-buffers out of a caller workspace, in a fixed order, so
// the *_workspace_size functions and the calls agree by construction.
struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *b) : base((char *)b) {}
    template <typename T> T *take(size_t count)
    {
        T *p = base ? (T *)(base + off) : nullptr;
        off += align_up(count * sizeof(T));
        return p;
    }
};

// Scalars at the front of every workspace.
struct Scalars {
    unsigned *status;     // 4 words
    double *d;            // 8 doubles
    double *partials;     // 2048 doubles
};

Scalars carve_scalars(Carver &c)
{
    Scalars s;
    s.status = c.take<unsigned>(4);
    s.d = c.take<double>(8);
    s.partials = c.take<double>(2048);
    return s;
}

int read_status(const unsigned *dev_status, hipStream_t stream, unsigned *out)
{
    unsigned h = 0;
    GQ_HIP(hipMemcpyAsync(&h, dev_status, sizeof(unsigned), hipMemcpyDeviceToHost, stream),
           "status readback");
    GQ_HIP(hipStreamSynchronize(stream), "stream synchronize");
    *out = h;
    return GQ_OK;
}

int status_to_code(unsigned st)
{
    if (st & ST_NONFINITE) return fail(GQ_ERR_NONFINITE, "non-finite value in an input");
    if (st & ST_NO_CALIB) return fail(GQ_ERR_NO_CALIBRATION, "mean(diag H) is not positive: no calibration data");
    if (st & ST_NOT_PD) return fail(GQ_ERR_NOT_PD, "damped Hessian is not positive definite (Cholesky pivot <= 0)");
    return GQ_OK;
}

GemmDesc gemm(const void *A, int64_t lda, const void *B, int64_t ldb, int64_t M, int64_t N, int64_t Kd,
              void *out, int64_t ldo)
{
    GemmDesc d{};
    d.A = A; d.lda = lda; d.B = B; d.ldb = ldb;
    d.M = M; d.N = N; d.Kd = Kd;
    d.out = out; d.ldo = ldo;
    d.out_t = nullptr; d.cin = nullptr; d.ldc = ldo;
    d.alpha = 1.0; d.beta = 0.0;
    d.alpha_dev = nullptr; d.alpha_pow = 0; d.beta_dev = nullptr; d.beta_pow = 0;
    d.tri = 0; d.mode = TILE_RECT;
    return d;
}


// ------------------------------------------------------------- sign iteration
// Scaled Newton-Schulz for sign(X), X symmetric with spectrum in [-1, 1]:
//   X <- a_k X + b_k X^3,  a_k = 1.5 alpha_k, b_k = -0.5 alpha_k^3,
//   alpha_k = sqrt(3 / (1 + l + l^2)),  l <- a_k l + b_k l^3.
// alpha_k maps [l, 1] onto [l', 1] with equal values at both ends, so every
// eigenvalue with |lambda| >= l_0 (relative to the bound) converges to +-1.
// The schedule stops once l > 1 - 1e-9: 20 iterations from 3e-7.  The last
// one matters less for the eigenvalues above l_0 (already within 3.3e-8 of
// +-1) than for those just below it, which it multiplies by 1.5 on their way
// to +-1.
//
// An eigenvalue lambda < 0 below the converged band leaves P with the
// eigenvalue lambda (1 + s) / 2, s = the iteration's value there, not 0.  Over
// the whole band the most negative such value is at most 0.036 l_0 b (b = the
// spectral bound the iteration is scaled by; 7.95e-9 b from l_0 = 3e-7,
// 3.3e-10 b from 1e-8: the schedule's polynomial evaluated on the real line).
// The projection must keep every eigenvalue above -1e-6 mean(diag H)
// (hipfire-calib-data, "The fix": the PSD bar), so the schedule starts at
// l_0 = min(3e-7, 2e-5 mean(diag H) / b), a floor of at most -7.2e-7
// mean(diag H): heavy-tailed Hessians, whose bound is a thousand times their
// mean diagonal, get three more iterations; a bound below 67 times it, none.
constexpr double kSignL0 = 3e-7;
constexpr double kSignL0Min = 1e-12;
constexpr double kSignFloor = 2e-5;
constexpr double kSignTol = 1e-9;

double sign_start(double mu, double bound)
{
    if (!(mu > 0.0) || !(bound > 0.0) || !std::isfinite(mu) || !std::isfinite(bound)) return kSignL0;
    return std::max(kSignL0Min, std::min(kSignL0, kSignFloor * mu / bound));
}

std::vector<double> sign_schedule(double l0 = kSignL0)
{
    std::vector<double> alphas;
    double l = l0;
    while (l < 1.0 - kSignTol && alphas.size() < 64) {
        const double a = std::sqrt(3.0 / (1.0 + l + l * l));
        alphas.push_back(a);
        l = 1.5 * a * l - 0.5 * a * a * a * l * l * l;
    }
    return alphas;
}

// Products of psd_project: emulated in integers on the int8 matrix cores below
// this order (exact int32 sums need K 128^2 < 2^31; beta stays >= 46), fp64
// matrix-core products at and above it.
constexpr int64_t kOzMaxK = 65536;
// Product kind chosen by gq_set_psd_products on this thread (GQ_PSD_*).
thread_local int g_psd_kind = GQ_PSD_AUTO;
// Sweep state chosen by gq_set_sweep_state on this thread (GQ_SWEEP_*).
thread_local int g_sweep_kind = GQ_SWEEP_AUTO;
bool psd_emulated(int64_t K) { return K < kOzMaxK && g_psd_kind != GQ_PSD_F64; }

struct PsdWs {
    Scalars sc;
    double *H64, *X, *Y, *Xn;
    double *partials;          // stream-K split-tile accumulators (fp64 path, large K)
    unsigned *flags;           // stream-K boundary counters
    int8_t *RH, *RX, *RY;      // split forms of H, the iterate X and Y0 / Z (emulated path)
    uint8_t *Cres;             // residues of one product
    int *eH;                   // row exponents of H's split form
    unsigned long long *hmax;  // largest magnitude of each row of H (fp64 bits)
};

PsdWs carve_psd(Carver &c, int64_t K, bool emulated)
{
    PsdWs w{};
    w.sc = carve_scalars(c);
    const size_t n = (size_t)K * (size_t)K;
    w.H64 = c.take<double>(n);
    w.Xn = c.take<double>(n);
    if (emulated) {
        const size_t pb = oz_planes_bytes(K);
        w.RH = c.take<int8_t>(pb);
        w.RX = c.take<int8_t>(pb);
        w.RY = c.take<int8_t>(pb);
        w.Cres = c.take<uint8_t>(pb);
        w.eH = c.take<int>((size_t)oz_padded(K));
        w.hmax = c.take<unsigned long long>((size_t)K);
    } else {
        w.X = c.take<double>(n);
        w.Y = c.take<double>(n);
        const bool sk = streamk_lower_worthwhile(K);
        w.partials = sk ? c.take<double>(streamk_partials_bytes(sizeof(double)) / sizeof(double)) : nullptr;
        w.flags = sk ? c.take<unsigned>(kStreamKMaxWorkers) : nullptr;
    }
    return w;
}

// Optional per-kernel timing of psd_project (gq_set_timing).
struct PsdTiming {
    bool on = false, valid = false;
    std::vector<hipEvent_t> ev;
    int launches = 0;
    double ms = 0.0;
    const char *kernel = "";
};
thread_local PsdTiming g_timing;

// Per panel: 1 / R_kk of its diagonal block.
constexpr int64_t kRinvPerPanel = kPanel;

struct FactorWs {
    Scalars sc;
    double *M, *X, *rinv;
};

FactorWs carve_factor(Carver &c, int64_t K)
{
    FactorWs w;
    w.sc = carve_scalars(c);
    const size_t n = (size_t)K * (size_t)K;
    const size_t nblk = (size_t)((K + kPanel - 1) / kPanel);
    w.M = c.take<double>(n);
    w.X = c.take<double>(n);
    w.rinv = c.take<double>(nblk * kRinvPerPanel);
    return w;
}

struct SweepWs {
    Scalars sc;
    float *Wk, *ET;
};

SweepWs carve_sweep(Carver &c, int64_t N, int64_t K)
{
    SweepWs w;
    w.sc = carve_scalars(c);
    w.Wk = c.take<float>((size_t)N * (size_t)K);
    // errors of two groups, k-major: a group's rows stay until the side stream's
    // update has read them, which ends before the group after next is swept
    w.ET = c.take<float>((size_t)2 * kSweepSuper * (size_t)N);
    return w;
}

// Enough for either kind of product when both are possible, so that the size
// does not depend on gq_set_psd_products.
size_t psd_bytes(int64_t K)
{
    Carver c(nullptr);
    carve_psd(c, K, false);
    if (K >= kOzMaxK) return c.off;
    Carver e(nullptr);
    carve_psd(e, K, true);
    return std::max(c.off, e.off);
}

size_t factor_bytes(int64_t K)
{
    Carver c(nullptr);
    carve_factor(c, K);
    return c.off;
}

size_t sweep_bytes(int64_t N, int64_t K)
{
    Carver c(nullptr);
    carve_sweep(c, N, K);
    return c.off;
}

// The public flags map onto the kernels' mode bits.
int mode_of(uint32_t flags)
{
    return ((flags & GQ_STATIC_GROUPS) ? MODE_STATIC : 0) | ((flags & GQ_NF4) ? MODE_NF4 : 0);
}

bool valid_group(int64_t G, int64_t K)
{
    if (G < 1 || G > 128) return false;
    if ((G & (G - 1)) != 0) return false;       // divides 128 <=> power of two <= 128
    return K % G == 0;
}

int check_sweep_args(const void *codes, const void *scales, const void *W, const void *U, int64_t N,
                     int64_t K, int64_t G)
{
    if (!codes || !scales || !W || !U) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (N < 1) return fail(GQ_ERR_INVALID_ARG, "N must be >= 1");
    if (K < 2 || (K & 1)) return fail(GQ_ERR_INVALID_ARG, "K must be even and >= 2 (two codes per byte)");
    if (!valid_group(G, K))
        return fail(GQ_ERR_INVALID_ARG, "group must be a power of two <= 128 that divides K");
    return GQ_OK;
}

// Upper Cholesky of the reversed, damped H, then the inverse; writes U (fp32).
int run_factor(float *U, const float *H, int64_t K, float damp, FactorWs &w, hipStream_t s)
{
    GQ_HIP(launch_fill_u32(w.sc.status, 4, 0u, s), "fill");
    double *mu = w.sc.d;
    GQ_HIP(launch_diag_mean_check(mu, H, K, w.sc.status, s), "diag mean");
    GQ_HIP(launch_damp_reverse(w.M, H, K, (double)damp, mu, s), "damp/reverse");
    const int64_t nblk = (K + kPanel - 1) / kPanel;
    Lookahead *la = nullptr;
    GQ_HIP(lookahead_for_current_device(&la), "lookahead stream");
    // The triangular inverse X = L^-1 (L = R^T, stored below M's diagonal) is
    // built on a third stream while the factorisation proceeds, block row by
    // block row from the top (right-looking forward substitution of L X = I,
    // X starting as I): once panel p is solved, its column block of L is final,
    // so X_p = L_pp^-1 X_p and then X_k -= L_kp X_p for the rows k below,
    // restricted to the columns left of the next panel (X_p is zero beyond).
    GQ_HIP(hipEventRecord(la->to_inv, s), "record");
    GQ_HIP(hipStreamWaitEvent(la->inv, la->to_inv, 0), "wait");
    GQ_HIP(launch_set_identity_f64(w.X, K, la->inv), "identity");
    // (the caller has recorded to_inv on s once panel p is solved)
    auto inverse_rows = [&](int64_t p) -> hipError_t {
        const int64_t q0 = p * kPanel;
        const int nbq = (int)((K - q0) < kPanel ? (K - q0) : kPanel);
        const int64_t q1 = q0 + nbq;
        hipError_t e = hipStreamWaitEvent(la->inv, la->to_inv, 0);
        if (e != hipSuccess) return e;
        // X_p = L_pp^-1 X_p = R_pp^-T X_p, in place, over the columns < q1
        e = launch_trsm_rt(w.M, K, q0, nbq, w.rinv + p * kRinvPerPanel, w.X + q0 * K, K, w.X + q0 * K, K, nullptr, 0, q1,
                           la->inv);
        if (e != hipSuccess || q1 >= K) return e;
        // X_k -= L_kp X_p for rows k >= q1, columns < q1; L_kp[k][b] = R[q0 + b][k]
        GemmDesc u = gemm(w.M + q0 * K + q1, K, w.X + q0 * K, K, K - q1, q1, nbq, w.X + q1 * K, K);
        u.cin = w.X + q1 * K;
        u.alpha = -1.0;
        u.beta = 1.0;
        return gemm_tn_f64(u, la->inv);
    };
    // Right-looking blocked Cholesky with a look-ahead of one panel.  Once the
    // block row of panel p+1 has its update from panel p, the diagonal block p+1
    // is factored right behind it on the caller's stream, while the rest of the
    // trailing update of panel p runs on the side stream.  The diagonal kernel
    // (one workgroup holding its block in LDS) thus reaches the hardware before
    // the large update's workgroups fill every CU, instead of waiting for one to
    // drain.  The block row of panel p+2 needs that update before its own, so
    // the next block-row update waits for the side stream.
    GQ_HIP(launch_potrf_diag(w.M, K, 0, (int)(K < kPanel ? K : kPanel), w.rinv, w.sc.status, s), "potrf diag");
    bool side_pending = false;
    for (int64_t p = 0; p < nblk; ++p) {
        const int64_t p0 = p * kPanel;
        const int nbp = (int)((K - p0) < kPanel ? (K - p0) : kPanel);
        const int64_t p1 = p0 + nbp;
        if (p1 >= K) {
            GQ_HIP(hipEventRecord(la->to_inv, s), "record");
            GQ_HIP(inverse_rows(p), "inverse rows");
            break;
        }
        // panel rows: R_{p,rest} = R_pp^{-T} A_{p,rest}, mirrored below the diagonal
        GQ_HIP(launch_trsm_rt(w.M, K, p0, nbp, w.rinv + p * kRinvPerPanel, w.M + p0 * K + p1, K, w.M + p0 * K + p1, K,
                              w.M + p1 * K + p0, K, K - p1, s),
               "trsm");
        // trailing update of the upper triangle, A_rest -= R_{p,rest}^T R_{p,rest}:
        // first the block row of panel p+1 (which has panel p-1's update once the
        // side stream's last product is done) ...
        const int nbn = (int)((K - p1) < kPanel ? (K - p1) : kPanel);
        const int64_t p2 = p1 + nbn;
        if (side_pending) GQ_HIP(hipStreamWaitEvent(s, la->to_main, 0), "wait trailing update");
        GemmDesc un = gemm(w.M + p0 * K + p1, K, w.M + p0 * K + p1, K, nbn, K - p1, nbp, w.M + p1 * K + p1, K);
        un.cin = w.M + p1 * K + p1;
        un.alpha = -1.0;
        un.beta = 1.0;
        un.tri = 2;
        GQ_HIP(gemm_tn_f64(un, s), "syrk next row");
        // ... then the rest on the side stream, and the inverse's rows of panel
        // p on the third, both behind one event: each event operation on s
        // lengthens the chain of dependent launches ...
        GQ_HIP(hipEventRecord(la->to_inv, s), "record");
        side_pending = p2 < K;
        if (side_pending) {
            GQ_HIP(hipStreamWaitEvent(la->side, la->to_inv, 0), "wait block row");
            GemmDesc u = gemm(w.M + p0 * K + p2, K, w.M + p0 * K + p2, K, K - p2, K - p2, nbp,
                              w.M + p2 * K + p2, K);
            u.cin = w.M + p2 * K + p2;
            u.alpha = -1.0;
            u.beta = 1.0;
            u.mode = TILE_UPPER;
            u.tri = 2;
            GQ_HIP(gemm_tn_f64(u, la->side), "syrk");
            GQ_HIP(hipEventRecord(la->to_main, la->side), "record");
        }
        GQ_HIP(inverse_rows(p), "inverse rows");
        // ... while the diagonal block of panel p+1 is factored here
        GQ_HIP(launch_potrf_diag(w.M, K, p1, nbn, w.rinv + (p + 1) * kRinvPerPanel, w.sc.status, s), "potrf diag");
    }
    if (side_pending) GQ_HIP(hipStreamWaitEvent(s, la->to_main, 0), "wait trailing update");
    GQ_HIP(hipEventRecord(la->inv_done, la->inv), "record");
    GQ_HIP(hipStreamWaitEvent(s, la->inv_done, 0), "wait inverse");
    // U = J R^-T J = J L^-1 J: U[i][j] = X[K-1-i][K-1-j]
    if (U) GQ_HIP(launch_flip(U, w.X, K, s), "flip");
    return GQ_OK;
}

// Act order's buffers: the permutation, its inverse, each permuted column's
// original group, and the codes in permuted column order.
struct ActOrder {
    int *perm, *inv, *gidx;
    uint8_t *cperm;
};

int run_sweep(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *U,
              const float *imp, int64_t N, int64_t K, int64_t G, int mode, SweepWs &w, hipStream_t s,
              const ActOrder *act = nullptr)
{
    GQ_HIP(launch_fill_u32(w.sc.status, 4, 0u, s), "fill");
    if (act)
        GQ_HIP(launch_gather_cols(w.Wk, W, act->perm, N, K, w.sc.status, s), "permute W");
    else
        GQ_HIP(launch_copy_check(w.Wk, W, N * K, w.sc.status, s), "copy W");
    uint8_t *const sweep_codes = act ? act->cperm : codes;
    if (imp) GQ_HIP(launch_check_finite(imp, K, w.sc.status, s), "check imp");
    // static groups: every scale from the original weights, before the sweep
    // (the round-to-nearest pass writes them; its codes are overwritten below)
    if (mode & MODE_STATIC)
        GQ_HIP(launch_rtn(W, codes, scales, nullptr, nullptr, N, K, G, mode, w.sc.status, s, nullptr), "scales");
    // Column order as in the unblocked sweep; every column receives the
    // feedback of all earlier columns before it is quantised: from its own
    // block inside the sweep kernel, from earlier blocks of its group through
    // the per-block products, and from earlier groups through the group
    // products.  Once group j is swept, its errors go into the next group on
    // this stream and into every later column on the side stream, one large
    // product that overlaps the next group's sweep (disjoint columns, finished
    // error rows); this stream waits for it only before it updates those
    // columns itself.
    Lookahead *la = nullptr;
    GQ_HIP(lookahead_for_current_device(&la), "lookahead stream");
    bool side_pending = false;
    auto update = [&](const float *Eg, int64_t k0, int64_t k1, int64_t c0, int64_t c1,
                      hipStream_t st) -> hipError_t {
        // Wk[:, c0:c1] -= E[k0:k1]^T U[k0:k1, c0:c1], E's rows k0.. at Eg
        GemmDesc d = gemm(Eg, N, U + k0 * K + c0, K, N, c1 - c0, k1 - k0, w.Wk + c0, K);
        d.cin = w.Wk + c0;
        d.alpha = -1.0;
        d.beta = 1.0;
        return gemm_tn_f32(d, st);
    };
    for (int64_t g0 = 0; g0 < K; g0 += kSweepSuper) {
        const int64_t g1 = (K - g0) < kSweepSuper ? K : g0 + kSweepSuper;
        float *const ETg = w.ET + ((g0 / kSweepSuper) & 1) * (int64_t)kSweepSuper * N;   // this group's E^T
        for (int64_t b0 = g0; b0 < g1; b0 += kSweepBlock) {
            const int64_t bw = (g1 - b0) < kSweepBlock ? (g1 - b0) : kSweepBlock;
            float *ETb = ETg + (b0 - g0) * N;          // this block's rows of E^T
            GQ_HIP(launch_sweep_block(w.Wk, ETb, sweep_codes, scales, U, N, K, G, b0, mode,
                                      act ? act->gidx : nullptr, s),
                   "sweep block");
            const int64_t e = b0 + bw;
            if (e < g1) {
                GemmDesc d = gemm(ETb, N, U + b0 * K + e, K, N, g1 - e, bw, w.Wk + e, K);
                d.cin = w.Wk + e;
                d.alpha = -1.0;
                d.beta = 1.0;
                GQ_HIP(gemm_tn_f32(d, s), "block update");
            }
        }
        if (g1 < K) {
            const int64_t n1 = (K - g1) < kSweepSuper ? K : g1 + kSweepSuper;   // the next group's end
            if (side_pending) {
                GQ_HIP(hipStreamWaitEvent(s, la->to_main, 0), "wait side update");
                side_pending = false;
            }
            if (n1 < K) {
                GQ_HIP(hipEventRecord(la->to_side, s), "record");
                GQ_HIP(hipStreamWaitEvent(la->side, la->to_side, 0), "wait group swept");
                GQ_HIP(update(ETg, g0, g1, n1, K, la->side), "group update (later groups)");
                GQ_HIP(hipEventRecord(la->to_main, la->side), "record");
                side_pending = true;
            }
            GQ_HIP(update(ETg, g0, g1, g1, n1, s), "group update (next group)");
        }
    }
    if (side_pending) GQ_HIP(hipStreamWaitEvent(s, la->to_main, 0), "wait side update");
    if (act) GQ_HIP(launch_unpermute_codes(codes, act->cperm, act->inv, N, K, s), "unpermute codes");
    if (qerr_out) {
        int64_t nparts = 0;
        GQ_HIP(launch_qerr(w.sc.partials, W, codes, scales, imp, N, K, G, mode, s, &nparts), "qerr");
        GQ_HIP(launch_qerr_reduce(w.sc.d, w.sc.partials, nparts, s), "qerr reduce");
    }
    unsigned st = 0;
    int rc = read_status(w.sc.status, s, &st);
    if (rc) return rc;
    rc = status_to_code(st);
    if (rc) return rc;
    if (qerr_out) {
        double nd[2] = {0.0, 0.0};
        GQ_HIP(hipMemcpyAsync(nd, w.sc.d, sizeof(nd), hipMemcpyDeviceToHost, s), "qerr readback");
        GQ_HIP(hipStreamSynchronize(s), "stream synchronize");
        *qerr_out = nd[1] > 0.0 ? std::sqrt(nd[0] / nd[1]) : 0.0;
    }
    return GQ_OK;
}

// gptq_quantize's sweep with U, the working weights and the errors in fp64
// (sweep64.hip), for the plain grid: the same column order and lazy blocks as
// run_sweep, every block and group update an fp64 product, all on the
// caller's stream.  U64 is the upper factor in fp64, W64 N x K doubles of
// scratch; the errors of one group (kSweepSuper x N doubles) reuse w.ET.
int run_sweep64(uint8_t *codes, float *scales, double *qerr_out, const float *W, const double *U64,
                const float *imp, int64_t N, int64_t K, int64_t G, SweepWs &w, double *W64, hipStream_t s)
{
    GQ_HIP(launch_fill_u32(w.sc.status, 4, 0u, s), "fill");
    GQ_HIP(launch_w64(W64, W, N * K, w.sc.status, s), "copy W");
    if (imp) GQ_HIP(launch_check_finite(imp, K, w.sc.status, s), "check imp");
    double *const ET = (double *)w.ET;
    auto update = [&](const double *Eb, int64_t k0, int64_t k1, int64_t c0, int64_t c1) -> hipError_t {
        // W64[:, c0:c1] -= E[k0:k1]^T U[k0:k1, c0:c1], E's rows k0.. at Eb
        GemmDesc d = gemm(Eb, N, U64 + k0 * K + c0, K, N, c1 - c0, k1 - k0, W64 + c0, K);
        d.cin = W64 + c0;
        d.alpha = -1.0;
        d.beta = 1.0;
        return gemm_tn_f64(d, s);
    };
    for (int64_t g0 = 0; g0 < K; g0 += kSweepSuper) {
        const int64_t g1 = (K - g0) < kSweepSuper ? K : g0 + kSweepSuper;
        for (int64_t b0 = g0; b0 < g1; b0 += kSweepBlock) {
            const int64_t bw = (g1 - b0) < kSweepBlock ? (g1 - b0) : kSweepBlock;
            double *ETb = ET + (b0 - g0) * N;
            GQ_HIP(launch_sweep64_block(W64, ETb, codes, scales, U64, N, K, G, b0, s), "sweep block");
            if (b0 + bw < g1) GQ_HIP(update(ETb, b0, b0 + bw, b0 + bw, g1), "block update");
        }
        if (g1 < K) GQ_HIP(update(ET, g0, g1, g1, K), "group update");
    }
    if (qerr_out) {
        int64_t nparts = 0;
        GQ_HIP(launch_qerr(w.sc.partials, W, codes, scales, imp, N, K, G, 0, s, &nparts), "qerr");
        GQ_HIP(launch_qerr_reduce(w.sc.d, w.sc.partials, nparts, s), "qerr reduce");
    }
    unsigned st = 0;
    int rc = read_status(w.sc.status, s, &st);
    if (rc) return rc;
    rc = status_to_code(st);
    if (rc) return rc;
    if (qerr_out) {
        double nd[2] = {0.0, 0.0};
        GQ_HIP(hipMemcpyAsync(nd, w.sc.d, sizeof(nd), hipMemcpyDeviceToHost, s), "qerr readback");
        GQ_HIP(hipStreamSynchronize(s), "stream synchronize");
        *qerr_out = nd[1] > 0.0 ? std::sqrt(nd[0] / nd[1]) : 0.0;
    }
    return GQ_OK;
}

// Whether gptq_quantize's sweep keeps its state in fp64: by default for the
// plain grid above K = 8192, where the fp32 state's drift decides measurably
// many rounding ties the other way from an fp64 sweep.
constexpr int64_t kSweep64MinK = 8193;
bool sweep64_applies(int64_t K, uint32_t flags)
{
    if (flags != 0u || g_sweep_kind == GQ_SWEEP_F32) return false;
    return g_sweep_kind == GQ_SWEEP_F64 || K >= kSweep64MinK;
}

// Workspace of gptq_sweep_f64: the sweep's (scalars, and errors of two fp32
// groups, i.e. one fp64 group), then the N x K fp64 working weights.
size_t sweep64_bytes(int64_t N, int64_t K)
{
    return sweep_bytes(N, K) + align_up((size_t)N * (size_t)K * sizeof(double));
}

}  // namespace

// The message gq_last_error returns, set by the other translation units (hfqm.hip).
int gq::set_error(int status, const char *msg)
{
    g_last_error = msg ? msg : "";
    return status;
}

extern "C" {

int gq_abi_version(void) { return GQ_ABI_VERSION; }

void gq_set_timing(int on) { g_timing.on = on != 0; }

int gq_set_psd_products(int kind)
{
    g_last_error.clear();
    if (kind != GQ_PSD_AUTO && kind != GQ_PSD_F64) return fail(GQ_ERR_INVALID_ARG, "unknown product kind");
    g_psd_kind = kind;
    return GQ_OK;
}

int gq_set_sweep_state(int kind)
{
    g_last_error.clear();
    if (kind != GQ_SWEEP_AUTO && kind != GQ_SWEEP_F32 && kind != GQ_SWEEP_F64)
        return fail(GQ_ERR_INVALID_ARG, "unknown sweep state");
    g_sweep_kind = kind;
    return GQ_OK;
}

int psd_project_last_timing(int *launches, double *product_ms, const char **kernel)
{
    g_last_error.clear();
    if (!g_timing.valid) return fail(GQ_ERR_INVALID_ARG, "no timed psd_project call on this thread");
    if (launches) *launches = g_timing.launches;
    if (product_ms) *product_ms = g_timing.ms;
    if (kernel) *kernel = g_timing.kernel;
    return GQ_OK;
}

const char *gq_last_error(void) { return g_last_error.c_str(); }

int hessian_accumulate(float *H, const void *X, int x_dtype, int64_t T, int64_t K, hipStream_t stream)
{
    g_last_error.clear();
    if (!H || (!X && T > 0)) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1 || T < 0) return fail(GQ_ERR_INVALID_ARG, "need K >= 1 and T >= 0");
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return fail(GQ_ERR_INVALID_ARG, "unknown x_dtype");
    if (T == 0) return GQ_OK;
    if (x_dtype == GQ_BF16) {
        GQ_HIP(launch_gram_bf16(H, (const uint16_t *)X, T, K, stream), "gram bf16");
    } else {
        GemmDesc d = gemm(X, K, X, K, K, K, T, H, K);
        d.cin = H;
        d.beta = 1.0;
        d.mode = TILE_LOWER;
        d.tri = 1;
        GQ_HIP(gemm_tn_f32(d, stream), "gram f32");
    }
    return GQ_OK;
}

}  // extern "C"

namespace {
// Splits per tile for a group of n chunks: the split count that best fills the
// chip's compute units with equal workgroups (tiles x splits against whole
// rounds of CUs, times the balance of chunks over splits), with a small charge
// per split for the partial tiles it writes and reads back.
int gram_splits(int64_t K, int64_t n, int ncu)
{
    if (n <= 1 || ncu <= 0) return 1;
    const int64_t tiles = gram_tiles(K);
    int best = 1;
    double best_eff = -1.0;
    for (int sp = 1; sp <= (int)std::min<int64_t>(n, 64); ++sp) {
        const int64_t wg = tiles * sp;
        const double fill = (double)wg / (double)(((wg + ncu - 1) / ncu) * ncu);
        const double bal = ((double)n / sp) / (double)((n + sp - 1) / sp);
        const double eff = fill * bal - 0.002 * sp;
        if (eff > best_eff + 1e-12) { best_eff = eff; best = sp; }
    }
    return best;
}

int device_cus(int *ncu)
{
    int dev = 0;
    GQ_HIP(hipGetDevice(&dev), "current device");
    GQ_HIP(hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    return GQ_OK;
}
}  // namespace

extern "C" {

size_t hessian_accumulate_chunks_workspace_size(int64_t K, int64_t n)
{
    if (K < 1 || n < 2) return 0;
    int ncu = 0;
    if (device_cus(&ncu) != GQ_OK) return 0;
    // the largest over the group sizes a call can form (chunks with T = 0 are
    // left out of a group)
    size_t need = 0;
    for (int64_t m = 2; m <= std::min<int64_t>(n, kGramMaxChunks); ++m)
        need = std::max(need, gram_split_bytes(K, gram_splits(K, m, ncu)));
    return need;
}

int hessian_accumulate_chunks(float *H, const void *const *X, const int64_t *T, int64_t n, int x_dtype, int64_t K,
                              void *ws, size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    if (!H || (n > 0 && (!X || !T))) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1 || n < 0) return fail(GQ_ERR_INVALID_ARG, "need K >= 1 and n >= 0");
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return fail(GQ_ERR_INVALID_ARG, "unknown x_dtype");
    bool dma = x_dtype == GQ_BF16 && K % 8 == 0;
    for (int64_t c = 0; c < n; ++c) {
        if (T[c] < 0) return fail(GQ_ERR_INVALID_ARG, "a chunk has T < 0");
        if (T[c] > 0 && !X[c]) return fail(GQ_ERR_INVALID_ARG, "null chunk pointer");
        if (T[c] > 0 && ((uintptr_t)X[c] & 15)) dma = false;
    }
    if (!dma) {
        // chunk by chunk, each added to H as hessian_accumulate does
        for (int64_t c = 0; c < n; ++c) {
            const int rc = hessian_accumulate(H, X[c], x_dtype, T[c], K, stream);
            if (rc) return rc;
        }
        return GQ_OK;
    }
    int ncu = 0;
    if (int rc = device_cus(&ncu)) return rc;
    for (int64_t c0 = 0; c0 < n; c0 += kGramMaxChunks) {
        GramChunks ch{};
        for (int64_t c = c0; c < n && c < c0 + kGramMaxChunks; ++c)
            if (T[c] > 0) {
                ch.x[ch.n] = (const uint16_t *)X[c];
                ch.t[ch.n] = T[c];
                ++ch.n;
            }
        if (ch.n == 0) continue;
        // the best split count whose partial tiles fit the workspace
        int splits = ws ? gram_splits(K, ch.n, ncu) : 1;
        while (splits > 1 && ws_bytes < gram_split_bytes(K, splits)) --splits;
        GQ_HIP(launch_gram_bf16_chunks(H, ch, K, splits, (float *)ws, stream), "gram bf16 chunks");
    }
    return GQ_OK;
}

size_t hessian_tril_bytes(int64_t K)
{
    if (K < 1) return 0;
    return (size_t)K * 4 + (size_t)K * (size_t)(K - 1) / 2 * 2;
}

int hessian_pack_tril(void *blob, const float *H, int64_t K, hipStream_t stream)
{
    g_last_error.clear();
    if (!blob || !H) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    GQ_HIP(launch_tril_pack((uint8_t *)blob, H, K, stream), "tril pack");
    return GQ_OK;
}

int hessian_unpack_tril(float *H, const void *blob, int64_t K, hipStream_t stream)
{
    g_last_error.clear();
    if (!blob || !H) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    GQ_HIP(launch_tril_unpack(H, (const uint8_t *)blob, K, stream), "tril unpack");
    return GQ_OK;
}

size_t psd_project_workspace_size(int64_t K) { return K < 1 ? 0 : psd_bytes(K); }

// One square for the bound, then (square, step) per iteration except the first,
// whose square is the bound's, then the rebuild: 2 * iterations + 1.
int psd_project_products(void) { return 2 * (int)sign_schedule().size() + 1; }

double psd_project_flops(int64_t K)
{
    if (K < 1) return 0.0;
    const double k = (double)K;
    return (double)psd_project_products() * k * k * (k + 1.0);
}

int psd_project(float *H, int64_t K, void *ws, size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    if (!H || !ws) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    if (ws_bytes < psd_bytes(K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    PsdWs w = carve_psd(cv, K, psd_emulated(K));
    const int64_t n = K * K;
    unsigned *status = w.sc.status;
    double *fro = w.sc.d + 0, *inv = w.sc.d + 1, *yfro = w.sc.d + 2, *c = w.sc.d + 3;
    double *c1inv = w.sc.d + 4, *c3inv = w.sc.d + 5;
    GQ_HIP(launch_fill_u32(status, 4, 0u, stream), "fill");
    if (w.flags) GQ_HIP(launch_fill_u32(w.flags, kStreamKMaxWorkers, 0u, stream), "fill");
    if (w.hmax) GQ_HIP(launch_fill_u32((unsigned *)w.hmax, 2 * K, 0u, stream), "fill");
    GQ_HIP(launch_sym_lower_to_f64(w.H64, H, K, status, stream, w.hmax), "symmetrise");
    GQ_HIP(launch_frobenius(fro, w.H64, n, w.sc.partials, stream), "norm");
    GQ_HIP(launch_scalar_combine(inv, fro, -1.0, nullptr, 0.0, stream), "inverse norm");
    // mean(diag H) for the schedule's start (its status word is a scratch word
    // that nobody reads: an all-zero H is projected, not refused)
    double *mu = w.sc.d + 6;
    GQ_HIP(launch_diag_mean_check(mu, H, K, status + 3, stream), "diag mean");
    std::vector<double> al;
    // once the bound is on the device: read it and mean(diag H) back and fix the
    // schedule (one small copy and a synchronisation, before the iterations)
    auto schedule = [&]() -> int {
        double hs[8];
        GQ_HIP(hipMemcpyAsync(hs, w.sc.d, sizeof(hs), hipMemcpyDeviceToHost, stream), "bound readback");
        GQ_HIP(hipStreamSynchronize(stream), "stream synchronize");
        // the spectrum of c * inv * H lies in [-1, 1]: the bound is 1 / (c * inv)
        al = sign_schedule(sign_start(hs[6], 1.0 / (hs[3] * hs[1])));
        return GQ_OK;
    };

    PsdTiming &tm = g_timing;
    const bool timing = tm.on;
    if (timing) {
        const size_t need = 2 * (2 * sign_schedule(kSignL0Min).size() + 1);   // the longest schedule
        while (tm.ev.size() < need) {
            hipEvent_t e;
            GQ_HIP(hipEventCreate(&e), "timing event");
            tm.ev.push_back(e);
        }
        tm.valid = false;
    }
    int launched = 0;
    auto mark = [&](bool before) -> hipError_t {
        if (!timing) return hipSuccess;
        return hipEventRecord(tm.ev[2 * launched + (before ? 0 : 1)], stream);
    };

    if (psd_emulated(K)) {
        // Products emulated exactly in integers (ozaki.hip).  H enters in its
        // row-scaled split form.  Every later operand is made, in split form
        // only, by the product before it:
        //   Y0 = (H / ||H||_F)^2                      (spectrum in [0, 1], exponent 1)
        //   X1 = a (c inv) H + b (c^3 inv) H Y0        (spectrum in [-1, 1], exponent 1)
        //   Z  = a I + b X^2                          (spectrum in [a + b, a], |a| < 2.6: exponent 2)
        //   X' = X Z                                  (= a X + b X^3)
        // so no fp64 iterate is stored.  The CRT writes only the K x K corner
        // of a split form (rounded up to 64 columns), so the rest of those
        // planes is cleared here once.
        const int beta = oz_beta(K);
        GQ_HIP(oz_clear_padding(w.RX, K, stream), "clear");
        GQ_HIP(oz_clear_padding(w.RY, K, stream), "clear");
        GQ_HIP(oz_split(w.H64, K, beta, w.RH, w.eH, stream, w.hmax), "split H");
        const OzOperand opH{w.RH, w.eH, 0}, opX{w.RX, nullptr, 1}, opY0{w.RY, nullptr, 1}, opZ{w.RY, nullptr, 2};
        auto product = [&](const GemmDesc &d, const OzOperand &A, const OzOperand &B, bool out_f32,
                           const OzOut &o) -> hipError_t {
            hipError_t e = mark(true);
            if (e == hipSuccess)
                e = oz_product(d, A, B, beta, w.Cres, out_f32, o, status, stream,
                               timing ? tm.ev[2 * launched + 1] : nullptr);
            ++launched;
            return e;
        };
        // Y0 (fp64 into Xn for its norm, split form into RY)
        GemmDesc y0 = gemm(nullptr, K, nullptr, K, K, K, K, w.Xn, K);
        y0.out_t = w.Xn;
        y0.alpha_dev = inv;
        y0.alpha_pow = 2;
        GQ_HIP(product(y0, opH, opH, false, OzOut{w.RY, 1, 0.0}), "sign square");
        GQ_HIP(launch_frobenius(yfro, w.Xn, n, w.sc.partials, stream), "norm");
        GQ_HIP(launch_scalar_combine(c, yfro, -0.5, nullptr, 0.0, stream), "bound");
        GQ_HIP(launch_scalar_combine(c1inv, c, 1.0, inv, 1.0, stream), "scalars");
        GQ_HIP(launch_scalar_combine(c3inv, c, 3.0, inv, 1.0, stream), "scalars");
        if (int rc = schedule()) return rc;
        for (size_t k = 0; k < al.size(); ++k) {
            const double a = 1.5 * al[k], b = -0.5 * al[k] * al[k] * al[k];
            if (k == 0) {
                GemmDesc st = gemm(nullptr, K, nullptr, K, K, K, K, nullptr, K);
                st.cin = w.H64;
                st.alpha = b;
                st.alpha_dev = c3inv;
                st.alpha_pow = 1;
                st.beta = a;
                st.beta_dev = c1inv;
                st.beta_pow = 1;
                GQ_HIP(product(st, opH, opY0, false, OzOut{w.RX, 1, 0.0}), "sign step");
                continue;
            }
            GemmDesc y = gemm(nullptr, K, nullptr, K, K, K, K, nullptr, K);
            y.alpha = b;
            GQ_HIP(product(y, opX, opX, false, OzOut{w.RY, 2, a}), "sign square");
            GemmDesc st = gemm(nullptr, K, nullptr, K, K, K, K, nullptr, K);
            GQ_HIP(product(st, opX, opZ, false, OzOut{w.RX, 1, 0.0}), "sign step");
        }
        // P = (H + sign(H) H) / 2, written to H as fp32 (both triangles)
        GemmDesc fin = gemm(nullptr, K, nullptr, K, K, K, K, H, K);
        fin.out_t = H;
        fin.cin = w.H64;
        fin.alpha = 0.5;
        fin.beta = 0.5;
        GQ_HIP(product(fin, opX, opH, true, OzOut{nullptr, 1, 0.0}), "projection");
    } else {
        auto product = [&](const GemmDesc &d, bool out_f32) -> hipError_t {
            hipError_t e = mark(true);
            if (e == hipSuccess)
                e = out_f32 ? gemm_tn_f64_out_f32_streamk(d, w.partials, w.flags, stream)
                            : gemm_tn_f64_streamk(d, w.partials, w.flags, stream);
            if (e == hipSuccess) e = mark(false);
            ++launched;
            return e;
        };
        // X0 = H / ||H||_F;  Y0 = X0^2;  c = ||Y0||_F^(-1/2) tightens the bound
        // (||H||_2 <= ||H^2||_F^(1/2)), so the spectrum of c X0 lies in [-1, 1].
        GemmDesc sq = gemm(w.H64, K, w.H64, K, K, K, K, w.Y, K);
        sq.alpha_dev = inv;
        sq.alpha_pow = 2;
        sq.mode = TILE_LOWER;
        sq.tri = 1;
        sq.out_t = w.Y;
        GQ_HIP(product(sq, false), "sign square");
        GQ_HIP(launch_frobenius(yfro, w.Y, n, w.sc.partials, stream), "norm");
        GQ_HIP(launch_scalar_combine(c, yfro, -0.5, nullptr, 0.0, stream), "bound");
        GQ_HIP(launch_scalar_combine(c1inv, c, 1.0, inv, 1.0, stream), "scalars");
        GQ_HIP(launch_scalar_combine(c3inv, c, 3.0, inv, 1.0, stream), "scalars");
        if (int rc = schedule()) return rc;
        double *X = w.X, *Xn = w.Xn;
        for (size_t k = 0; k < al.size(); ++k) {
            const double a = 1.5 * al[k], b = -0.5 * al[k] * al[k] * al[k];
            if (k == 0) {
                // X0 = inv H, so X1 = a (c inv) H + b (c^3 inv) H Y0
                GemmDesc st = gemm(w.H64, K, w.Y, K, K, K, K, X, K);
                st.cin = w.H64;
                st.alpha = b;
                st.alpha_dev = c3inv;
                st.alpha_pow = 1;
                st.beta = a;
                st.beta_dev = c1inv;
                st.beta_pow = 1;
                st.mode = TILE_LOWER;
                st.tri = 1;
                st.out_t = X;
                GQ_HIP(product(st, false), "sign step");
                continue;
            }
            GemmDesc y = gemm(X, K, X, K, K, K, K, w.Y, K);
            y.mode = TILE_LOWER;
            y.tri = 1;
            y.out_t = w.Y;
            GQ_HIP(product(y, false), "sign square");
            GemmDesc st = gemm(X, K, w.Y, K, K, K, K, Xn, K);
            st.cin = X;
            st.alpha = b;
            st.beta = a;
            st.mode = TILE_LOWER;
            st.tri = 1;
            st.out_t = Xn;
            GQ_HIP(product(st, false), "sign step");
            double *t = X;
            X = Xn;
            Xn = t;
        }
        // P = (H + sign(H) H) / 2, written to H as fp32 (both triangles)
        GemmDesc fin = gemm(X, K, w.H64, K, K, K, K, H, K);
        fin.cin = w.H64;
        fin.alpha = 0.5;
        fin.beta = 0.5;
        fin.mode = TILE_LOWER;
        fin.tri = 1;
        fin.out_t = H;
        GQ_HIP(product(fin, true), "projection");
    }
    unsigned st = 0;
    int rc = read_status(status, stream, &st);
    if (rc) return rc;
    if (timing) {
        double total = 0.0;
        for (int i = 0; i < launched; ++i) {
            float ms = 0.0f;
            GQ_HIP(hipEventElapsedTime(&ms, tm.ev[2 * i], tm.ev[2 * i + 1]), "timing");
            total += ms;
        }
        tm.launches = launched;
        tm.ms = total;
        tm.kernel = !psd_emulated(K) ? "gemm_tn_streamk_kernel<double,double> (fp64 products)"
                    : oz_mods(K) == 12 ? "oz_gemm_kernel (int8 residue products, 12 moduli)"
                                       : "oz_gemm_kernel (int8 residue products, 13 moduli)";
        tm.valid = true;
    }
    if (st & ST_RANGE) return fail(GQ_ERR_INTERNAL, "an iterate of the sign iteration left the range [-2, 2]");
    return status_to_code(st);
}

size_t gptq_factor_workspace_size(int64_t K) { return K < 1 ? 0 : factor_bytes(K); }

int gptq_factor(float *U, const float *H, int64_t K, float damp, void *ws, size_t ws_bytes,
                hipStream_t stream)
{
    g_last_error.clear();
    if (!U || !H || !ws) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    if (!(damp >= 0.0f) || !std::isfinite(damp)) return fail(GQ_ERR_INVALID_ARG, "damp must be finite and >= 0");
    if (ws_bytes < factor_bytes(K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    FactorWs w = carve_factor(cv, K);
    int rc = run_factor(U, H, K, damp, w, stream);
    if (rc) return rc;
    unsigned st = 0;
    rc = read_status(w.sc.status, stream, &st);
    if (rc) return rc;
    return status_to_code(st);
}

size_t gptq_sweep_workspace_size(int64_t N, int64_t K, int64_t group)
{
    (void)group;
    if (N < 1 || K < 1) return 0;
    return sweep_bytes(N, K);
}

int gptq_sweep_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *U,
                  const float *imp, int64_t N, int64_t K, int64_t group, uint32_t flags, void *ws,
                  size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    int rc = check_sweep_args(codes, scales, W, U, N, K, group);
    if (rc) return rc;
    if (flags & GQ_ACT_ORDER)
        return fail(GQ_ERR_INVALID_ARG, "act order needs the factor of the permuted Hessian: use gptq_quantize_ex");
    if (flags & ~(uint32_t)(GQ_STATIC_GROUPS | GQ_NF4)) return fail(GQ_ERR_INVALID_ARG, "unknown flag bits");
    if (!ws) return fail(GQ_ERR_INVALID_ARG, "null workspace");
    if (ws_bytes < sweep_bytes(N, K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    SweepWs w = carve_sweep(cv, N, K);
    return run_sweep(codes, scales, qerr_out, W, U, imp, N, K, group, mode_of(flags), w, stream);
}

int gptq_sweep(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *U,
               const float *imp, int64_t N, int64_t K, int64_t group, void *ws, size_t ws_bytes,
               hipStream_t stream)
{
    return gptq_sweep_ex(codes, scales, qerr_out, W, U, imp, N, K, group, 0u, ws, ws_bytes, stream);
}

void gq_nf4_levels(float *levels)
{
    if (levels)
        for (int i = 0; i < 16; ++i) levels[i] = kNF4[i];
}

struct RtnWs {
    Scalars sc;
    double *partials;                                  // rtn_partials(N, K) pairs
};

RtnWs carve_rtn(Carver &c, int64_t N, int64_t K)
{
    RtnWs w;
    w.sc = carve_scalars(c);
    w.partials = c.take<double>((size_t)2 * (size_t)rtn_partials(N, K));
    return w;
}

int hadamard_rotate_rows(float *A, int64_t rows, int64_t K, int64_t ld, int64_t block, const float *signs,
                         hipStream_t stream)
{
    g_last_error.clear();
    if (!A) return fail(GQ_ERR_INVALID_ARG, "null matrix");
    if (rows < 0 || K < 1 || ld < K) return fail(GQ_ERR_INVALID_ARG, "bad sizes");
    if (!hadamard_block_ok(K, block))
        return fail(GQ_ERR_INVALID_ARG, "block must be a power of two <= 4096 that divides K");
    GQ_HIP(launch_fwht_rows(A, rows, K, ld, block, signs, stream), "fwht rows");
    return GQ_OK;
}

size_t hadamard_rotate_hessian_workspace_size(int64_t K)
{
    if (K < 1) return 0;
    return align_up((size_t)K * (size_t)K * sizeof(float));
}

int hadamard_rotate_hessian(float *H, int64_t K, int64_t block, const float *signs, void *ws, size_t ws_bytes,
                            hipStream_t stream)
{
    g_last_error.clear();
    if (!H || !ws) return fail(GQ_ERR_INVALID_ARG, "null matrix or workspace");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    if (!hadamard_block_ok(K, block))
        return fail(GQ_ERR_INVALID_ARG, "block must be a power of two <= 4096 that divides K");
    if (ws_bytes < hadamard_rotate_hessian_workspace_size(K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    // H' = R H R^T: T = H R^T (each row of H rotated), and H' = R T = (T^T R^T)^T;
    // H' is symmetric, so it is T^T R^T itself: the rows of T^T rotated
    float *T = (float *)ws;
    GQ_HIP(launch_fwht_rows(H, K, K, K, block, signs, stream), "fwht rows");
    GQ_HIP(launch_transpose(T, H, K, stream), "transpose");
    if (launch_fwht_rows(H, K, K, K, block, signs, stream, T) == hipSuccess) return GQ_OK;   // T's rows into H
    (void)hipGetLastError();
    // small blocks or unaligned buffers: rotate in place, then copy back
    GQ_HIP(launch_fwht_rows(T, K, K, K, block, signs, stream), "fwht rows");
    GQ_HIP(hipMemcpyAsync(H, T, (size_t)K * (size_t)K * sizeof(float), hipMemcpyDeviceToDevice, stream), "copy");
    return GQ_OK;
}

size_t rtn_quantize_workspace_size(int64_t N, int64_t K, int64_t group)
{
    (void)group;
    if (N < 1 || K < 1) return 0;
    Carver c(nullptr);
    carve_rtn(c, N, K);
    return c.off;
}

static int check_rtn_args(const uint8_t *codes, const float *scales, const float *W, int64_t N, int64_t K,
                          int64_t group, uint32_t flags)
{
    if (flags & ~(uint32_t)(GQ_STATIC_GROUPS | GQ_NF4)) return fail(GQ_ERR_INVALID_ARG, "unknown flag bits");
    if (!codes || !scales || !W) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (N < 1) return fail(GQ_ERR_INVALID_ARG, "N must be >= 1");
    if (K < 2 || (K & 1)) return fail(GQ_ERR_INVALID_ARG, "K must be even and >= 2 (two codes per byte)");
    if (!valid_group(group, K))
        return fail(GQ_ERR_INVALID_ARG, "group must be a power of two <= 128 that divides K");
    return GQ_OK;
}

// The round-to-nearest pack over a workspace already carved (status word,
// qerr's scalars and partial sums); the status word is cleared first.
static int run_rtn(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp, int64_t N,
                   int64_t K, int64_t group, uint32_t flags, const RtnWs &w, hipStream_t stream)
{
    const int mode = mode_of(flags);
    GQ_HIP(launch_fill_u32(w.sc.status, 4, 0u, stream), "fill");
    if (imp) GQ_HIP(launch_check_finite(imp, K, w.sc.status, stream), "check imp");
    int64_t nparts = 0;
    GQ_HIP(launch_rtn(W, codes, scales, imp, qerr_out ? w.partials : nullptr, N, K, group, mode, w.sc.status,
                      stream, &nparts),
           "rtn");
    if (qerr_out) GQ_HIP(launch_qerr_reduce(w.sc.d, w.partials, nparts, stream), "qerr reduce");
    // status and the two sums come back with one synchronisation
    unsigned st = 0;
    double nd[2] = {0.0, 0.0};
    GQ_HIP(hipMemcpyAsync(&st, w.sc.status, sizeof(st), hipMemcpyDeviceToHost, stream), "status readback");
    if (qerr_out) GQ_HIP(hipMemcpyAsync(nd, w.sc.d, sizeof(nd), hipMemcpyDeviceToHost, stream), "qerr readback");
    GQ_HIP(hipStreamSynchronize(stream), "stream synchronize");
    const int rc = status_to_code(st);
    if (rc) return rc;
    if (qerr_out) *qerr_out = nd[1] > 0.0 ? std::sqrt(nd[0] / nd[1]) : 0.0;
    return GQ_OK;
}

int rtn_quantize_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp, int64_t N,
                    int64_t K, int64_t group, uint32_t flags, void *ws, size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    int rc = check_rtn_args(codes, scales, W, N, K, group, flags);
    if (rc) return rc;
    if (!ws) return fail(GQ_ERR_INVALID_ARG, "null workspace");
    if (ws_bytes < rtn_quantize_workspace_size(N, K, group)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    const RtnWs w = carve_rtn(cv, N, K);
    return run_rtn(codes, scales, qerr_out, W, imp, N, K, group, flags, w, stream);
}

int rtn_quantize(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp, int64_t N,
                 int64_t K, int64_t group, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return rtn_quantize_ex(codes, scales, qerr_out, W, imp, N, K, group, 0u, ws, ws_bytes, stream);
}

}  // extern "C"

// Scratch of rtn_quantize_noalloc, in place of a caller workspace: one copy per
// device, held until the process ends.  Its name is a host-side stand-in; the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[GQ_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void *> g_scratch;          // by device ordinal; nullptr until looked up

int scratch_for_current_device(void **out)
{
    int dev = 0;
    GQ_HIP(hipGetDevice(&dev), "current device");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((size_t)dev >= g_scratch.size()) g_scratch.resize((size_t)dev + 1, nullptr);
    if (!g_scratch[(size_t)dev]) {
        void *p = nullptr;
        GQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
        if (!p) return fail(GQ_ERR_HIP, "scratch address: null");
        g_scratch[(size_t)dev] = p;
    }
    *out = g_scratch[(size_t)dev];
    return GQ_OK;
}
}  // namespace

extern "C" {

int rtn_quantize_noalloc(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp,
                         int64_t N, int64_t K, int64_t group, uint32_t flags, hipStream_t stream)
{
    g_last_error.clear();
    int rc = check_rtn_args(codes, scales, W, N, K, group, flags);
    if (rc) return rc;
    if (rtn_quantize_workspace_size(N, K, group) > (size_t)GQ_NOALLOC_SCRATCH_BYTES)
        return fail(GQ_ERR_INVALID_ARG, "needs more scratch than the library's fixed scratch holds");
    void *ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc) return rc;
    Carver cv(ws);
    const RtnWs w = carve_rtn(cv, N, K);
    return run_rtn(codes, scales, qerr_out, W, imp, N, K, group, flags, w, stream);
}

int gptq_factor_f64(double *U, const float *H, int64_t K, float damp, void *ws, size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    if (!U || !H || !ws) return fail(GQ_ERR_INVALID_ARG, "null required pointer");
    if (K < 1) return fail(GQ_ERR_INVALID_ARG, "K must be >= 1");
    if (!(damp >= 0.0f) || !std::isfinite(damp)) return fail(GQ_ERR_INVALID_ARG, "damp must be finite and >= 0");
    if (ws_bytes < factor_bytes(K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    FactorWs w = carve_factor(cv, K);
    int rc = run_factor(nullptr, H, K, damp, w, stream);
    if (rc) return rc;
    GQ_HIP(launch_flip64(U, w.X, K, stream), "flip");
    unsigned st = 0;
    rc = read_status(w.sc.status, stream, &st);
    if (rc) return rc;
    return status_to_code(st);
}

size_t gptq_sweep_f64_workspace_size(int64_t N, int64_t K, int64_t group)
{
    (void)group;
    if (N < 1 || K < 1) return 0;
    return sweep64_bytes(N, K);
}

int gptq_sweep_f64(uint8_t *codes, float *scales, double *qerr_out, const float *W, const double *U,
                   const float *imp, int64_t N, int64_t K, int64_t group, void *ws, size_t ws_bytes,
                   hipStream_t stream)
{
    g_last_error.clear();
    int rc = check_sweep_args(codes, scales, W, U, N, K, group);
    if (rc) return rc;
    if (!ws) return fail(GQ_ERR_INVALID_ARG, "null workspace");
    if (ws_bytes < sweep64_bytes(N, K)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    Carver cv(ws);
    SweepWs w = carve_sweep(cv, N, K);
    double *W64 = (double *)((char *)ws + sweep_bytes(N, K));
    return run_sweep64(codes, scales, qerr_out, W, U, imp, N, K, group, w, W64, stream);
}

size_t gptq_quantize_workspace_size(int64_t N, int64_t K, int64_t group)
{
    (void)group;
    if (N < 1 || K < 1) return 0;
    // factor, U, sweep, and the fp64 sweep's working weights (present whatever
    // the sweep's state, so that the size does not depend on gq_set_sweep_state)
    return factor_bytes(K) + align_up((size_t)K * (size_t)K * sizeof(float)) + sweep_bytes(N, K) +
           align_up((size_t)N * (size_t)K * sizeof(double));
}

// Workspace of gptq_quantize_ex: gptq_quantize's, plus for act order the
// permuted H, the permutation's three int arrays and the permuted codes.
size_t act_bytes(int64_t N, int64_t K)
{
    return align_up((size_t)K * (size_t)K * sizeof(float)) + 3 * align_up((size_t)K * sizeof(int)) +
           align_up((size_t)N * (size_t)(K / 2));
}

size_t gptq_quantize_ex_workspace_size(int64_t N, int64_t K, int64_t group, uint32_t flags)
{
    if (N < 1 || K < 1) return 0;
    const size_t base = gptq_quantize_workspace_size(N, K, group);
    return (flags & GQ_ACT_ORDER) ? base + act_bytes(N, K) : base;
}

int gptq_quantize_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *H,
                     const float *imp, int64_t N, int64_t K, int64_t group, float damp, uint32_t flags, void *ws,
                     size_t ws_bytes, hipStream_t stream)
{
    g_last_error.clear();
    int rc = check_sweep_args(codes, scales, W, H, N, K, group);
    if (rc) return rc;
    if (flags & ~(uint32_t)(GQ_STATIC_GROUPS | GQ_NF4 | GQ_ACT_ORDER))
        return fail(GQ_ERR_INVALID_ARG, "unknown flag bits");
    if ((flags & GQ_ACT_ORDER) && !(flags & GQ_STATIC_GROUPS))
        return fail(GQ_ERR_INVALID_ARG, "act order needs static groups (the packed layout keeps contiguous groups)");
    if ((flags & GQ_ACT_ORDER) && K > INT32_MAX / 2) return fail(GQ_ERR_INVALID_ARG, "K too large for act order");
    if (flags & GQ_ACT_ORDER) {
        if (!ws) return fail(GQ_ERR_INVALID_ARG, "null workspace");
        if (ws_bytes < gptq_quantize_ex_workspace_size(N, K, group, flags))
            return fail(GQ_ERR_INVALID_ARG, "workspace too small");
        // columns by decreasing diag(H): permute H on both sides, factor it, and
        // sweep W's permuted columns with their original groups' static scales
        char *base = (char *)ws;
        const size_t fb = factor_bytes(K), ub = align_up((size_t)K * (size_t)K * sizeof(float));
        float *U = (float *)(base + fb);
        char *sweep_ws = base + fb + ub;
        Carver cv(sweep_ws + sweep_bytes(N, K) + align_up((size_t)N * (size_t)K * sizeof(double)));
        float *Hp = cv.take<float>((size_t)K * (size_t)K);
        ActOrder act;
        act.perm = cv.take<int>((size_t)K);
        act.inv = cv.take<int>((size_t)K);
        act.gidx = cv.take<int>((size_t)K);
        act.cperm = cv.take<uint8_t>((size_t)N * (size_t)(K / 2));
        GQ_HIP(launch_act_perm(act.perm, act.inv, act.gidx, H, K, group, stream), "act order");
        // U's buffer is free until the factor: it holds H's full symmetric copy
        GQ_HIP(launch_perm_sym(Hp, H, act.perm, U, K, stream), "permute H");
        rc = gptq_factor(U, Hp, K, damp, base, fb, stream);
        if (rc) return rc;
        Carver sc(sweep_ws);
        SweepWs w = carve_sweep(sc, N, K);
        return run_sweep(codes, scales, qerr_out, W, U, imp, N, K, group, mode_of(flags), w, stream, &act);
    }
    if (!ws) return fail(GQ_ERR_INVALID_ARG, "null workspace");
    if (ws_bytes < gptq_quantize_workspace_size(N, K, group)) return fail(GQ_ERR_INVALID_ARG, "workspace too small");
    char *base = (char *)ws;
    const size_t fb = factor_bytes(K);
    float *U = (float *)(base + fb);
    void *sweep_ws = base + fb + align_up((size_t)K * (size_t)K * sizeof(float));
    rc = gptq_factor(U, H, K, damp, base, fb, stream);
    if (rc) return rc;
    if (sweep64_applies(K, flags)) {
        // U in fp64 into the factor's M (free once the factor has returned),
        // from the same L^-1 the fp32 U was rounded from
        Carver fc(base);
        FactorWs fw = carve_factor(fc, K);
        GQ_HIP(launch_flip64(fw.M, fw.X, K, stream), "flip");
        Carver sc(sweep_ws);
        SweepWs w = carve_sweep(sc, N, K);
        double *W64 = (double *)((char *)sweep_ws + sweep_bytes(N, K));
        return run_sweep64(codes, scales, qerr_out, W, fw.M, imp, N, K, group, w, W64, stream);
    }
    return gptq_sweep_ex(codes, scales, qerr_out, W, U, imp, N, K, group, flags, sweep_ws, sweep_bytes(N, K),
                         stream);
}

int gptq_quantize(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *H,
                  const float *imp, int64_t N, int64_t K, int64_t group, float damp, void *ws,
                  size_t ws_bytes, hipStream_t stream)
{
    return gptq_quantize_ex(codes, scales, qerr_out, W, H, imp, N, K, group, damp, 0u, ws, ws_bytes, stream);
}

}  // extern "C"
