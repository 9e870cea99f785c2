/*
 * gq.h -- C ABI of the calibration-Hessian GPTQ int4 library for AMD MI355X
 * (gfx950).  Everything runs in hand-written HIP kernels; the library never
 * allocates or frees device memory: the caller owns every buffer and workspace.
 *
 * State the library keeps across calls
 *   - a thread-local error string (gq_last_error);
 *   - per host thread and device, two HIP streams (default priority,
 *     non-blocking) and four events, created on the first gptq_factor or
 *     gptq_sweep on that device and kept until the process ends.  Those calls
 *     fork part of their work onto the two streams (the Cholesky's trailing
 *     updates and the triangular inverse beside the panel chain; each sweep
 *     group's update of the later columns beside the next group's sweep), and
 *     join it back into the caller's stream with events before they
 *     synchronise it, so no work of a call is pending when it returns;
 *   - the testing and profiling settings at the end of this header
 *     (thread-local), and the HIP events timed psd_project calls record into
 *     (created when timing is first used on a thread);
 *   - one 64 KiB static device array per device (GQ_NOALLOC_SCRATCH_BYTES),
 *     part of the code object: the scratch of rtn_quantize_noalloc only.
 *   Nothing else: no device memory allocated at run time, no cache of inputs
 *   or results.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked "host".  Device buffers must be
 *     4-byte aligned; 16-byte alignment (what hipMalloc and PyTorch give) enables
 *     the vectorised paths.
 *   - Matrices are row-major.  H is K x K fp32.  A symmetric input is read from
 *     its lower triangle (row >= column) only.
 *   - Calls return a gq_status.  GQ_OK is 0; the detail of any other status is
 *     in gq_last_error() (thread-local, valid until the next call on the same
 *     host thread).  On an error the outputs are undefined.
 *   - hessian_* calls are asynchronous: they validate arguments, enqueue kernels
 *     and return; they report argument and launch errors only.  psd_project,
 *     gptq_factor, gptq_sweep and gptq_quantize synchronise their stream before
 *     returning, to report data-dependent status (and qerr).
 *   - Calls that share a workspace must not overlap on different streams.
 *   - New behaviour is added as new symbols that the old ones forward to, never
 *     by changing a signature (the extension rule of the ork-driver wiki page
 *     "Exp 2026-08-18 GPTQ Int4", qerr section).
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQ_ABI_VERSION 1

typedef enum gq_status {
    GQ_OK = 0,
    GQ_ERR_INVALID_ARG = 1,    /* bad size, null required pointer, short workspace   */
    GQ_ERR_NOT_PD = 2,         /* a Cholesky pivot of the damped Hessian was <= 0     */
    GQ_ERR_NONFINITE = 3,      /* NaN or Inf in W, in the lower triangle of H, or imp */
    GQ_ERR_NO_CALIBRATION = 4, /* mean(diag H) <= 0: refuse rather than guess         */
    GQ_ERR_HIP = 5,            /* a HIP runtime call failed                           */
    GQ_ERR_INTERNAL = 6,       /* an internal numerical invariant failed (a bug)      */
    GQ_ERR_IO = 7              /* a file could not be read or written, or is not a
                                  well-formed HFQM package                            */
} gq_status;

typedef enum gq_dtype { GQ_F32 = 0, GQ_BF16 = 1 } gq_dtype;

/* ABI version of the loaded library (GQ_ABI_VERSION of its build). */
int gq_abi_version(void);

/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char *gq_last_error(void);

/*
 * hessian_accumulate -- H_lower += X^T X for one activation chunk.
 *
 * The calibration Hessian is the full Gram matrix of the activations
 * (hipfire-calib-data dataset card, "Hessian storage": full Hessians, not
 * diagonals), and it is a sum over token chunks, so chunks accumulated in any
 * split add up to the single-pass statistic (AtomicChat Qwen3.8-27B GGUF page,
 * "The importance matrix").
 *
 *   H       K x K fp32, row-major.  Entries with row >= column are updated in
 *           place; the strict upper triangle is not touched.  The caller zeroes
 *           H before the first chunk.  Each call adds its chunk's sum, formed in
 *           fp32 accumulators, to H once.
 *   X       T x K row-major activations, fp32 (x_dtype GQ_F32) or bf16
 *           (GQ_BF16).  Not modified.
 *   T, K    tokens in this chunk (T >= 0; T == 0 is a no-op) and channels (K >= 1).
 *   stream  HIP stream for the launch.
 * Errors: GQ_ERR_INVALID_ARG for null pointers, K < 1, T < 0 or an unknown dtype.
 */
int hessian_accumulate(float *H, const void *X, int x_dtype, int64_t T, int64_t K,
                       hipStream_t stream);

/*
 * hessian_accumulate_chunks -- H_lower += sum over c of X_c^T X_c for n chunks in
 * one call: the same statistic as n hessian_accumulate calls, since it is a sum
 * over chunks (AtomicChat Qwen3.8-27B GGUF page, "The importance matrix").  For
 * bf16 chunks with K % 8 == 0 and 16-byte aligned pointers, up to 128 chunks go
 * into one launch whose workgroups each take one tile and a contiguous range of
 * chunks; with a workspace, several workgroups share a tile so that every
 * compute unit is busy, and their partial tiles are added to H in a fixed order
 * (the result does not depend on timing, and it may differ from n separate
 * calls in the rounding of the fp32 sums).  Other chunks run as n
 * hessian_accumulate calls.
 *   H     K x K fp32, lower triangle updated in place (as hessian_accumulate).
 *   X     host array of n device pointers, chunk c being T[c] x K row-major.
 *   T     host array of n token counts (>= 0; 0 skips the chunk).
 *   ws    device workspace of hessian_accumulate_chunks_workspace_size(K, n)
 *         bytes (a smaller one means fewer workgroups per tile), or NULL (one
 *         workgroup per tile).  The size query needs the current device.
 * Asynchronous, like hessian_accumulate.
 * Errors: GQ_ERR_INVALID_ARG (null pointers, K < 1, n < 0, T[c] < 0, unknown
 *         dtype), GQ_ERR_HIP.
 */
size_t hessian_accumulate_chunks_workspace_size(int64_t K, int64_t n);
int hessian_accumulate_chunks(float *H, const void *const *X, const int64_t *T, int64_t n, int x_dtype,
                              int64_t K, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of a Bf16TrilDiagF32 blob: K*4 + K*(K-1)/2*2 (hipfire-calib-data,
 * "Hessian storage: Bf16TrilDiagF32"). 0 for K < 1. */
size_t hessian_tril_bytes(int64_t K);

/*
 * hessian_pack_tril -- H -> Bf16TrilDiagF32 blob (hipfire-calib-data, "Hessian
 * storage: Bf16TrilDiagF32 (quant_type 130)"): K little-endian f32 words holding
 * the exact diagonal, then K*(K-1)/2 little-endian u16 words; word i*(i-1)/2 + j
 * (i > j) holds the top 16 bits of H[i][j] (truncation, f32_bits >> 16, not
 * rounding).  Only the lower triangle of H is read.
 *   blob  hessian_tril_bytes(K) bytes, written.    H  K x K fp32, read.
 * Errors: GQ_ERR_INVALID_ARG for null pointers or K < 1.
 */
int hessian_pack_tril(void *blob, const float *H, int64_t K, hipStream_t stream);

/*
 * hessian_unpack_tril -- Bf16TrilDiagF32 blob -> full symmetric H: H[i][i] is the
 * stored f32, H[i][j] = H[j][i] = f32(u16 << 16) (mirrored on read, same section).
 *   H     K x K fp32, written in full.    blob  hessian_tril_bytes(K) bytes, read.
 * Errors: GQ_ERR_INVALID_ARG for null pointers or K < 1.
 */
int hessian_unpack_tril(float *H, const void *blob, int64_t K, hipStream_t stream);

/* Workspace bytes psd_project needs for size K. */
size_t psd_project_workspace_size(int64_t K);

/* Floating-point operations psd_project executes for size K under its shortest
 * schedule (the method's cost; the dataset card's "The fix" prices the
 * eigendecomposition at O(K^3)): each symmetric K x K product of the sign
 * iteration counts K*K*(K+1) (the lower triangle it computes), plus the final
 * rebuild.  Host-only query. */
double psd_project_flops(int64_t K);

/* Number of symmetric products psd_project launches under its shortest
 * schedule, for any K (41).  A Hessian whose spectral bound is large against its
 * mean diagonal gets a few more (see psd_project); the testing section's
 * psd_project_last_timing reports the count of a given call.  Host-only query. */
int psd_project_products(void);

/*
 * psd_project -- H <- nearest positive-semidefinite matrix in Frobenius norm:
 * eigenvalues clipped at zero, rebuilt, symmetrised (hipfire-calib-data, "The
 * fix"; required before Cholesky on stored Hessians).  Computed on the device
 * without an eigendecomposition, as P = (H + sign(H) H) / 2 with sign(H) from a
 * scaled Newton-Schulz iteration.  Its schedule starts from the spectral bound
 * and mean(diag H), read back once, so that every eigenvalue of the result stays
 * above -1e-6 mean(diag H): 20 iterations (41 products) when the bound is
 * within about 67 times the mean diagonal, a few more when it is larger (three
 * at a thousand times).  For K < 65536 its symmetric products are
 * computed exactly in integers on the int8 matrix cores from operands rounded
 * to 40-bit integers up to K = 8192 and 43-44-bit integers above (one
 * power-of-two scale per row; residues modulo 12 or 13 moduli, Chinese
 * remainder reconstruction, one rounding to fp64); from K = 65536 on,
 * fp64 matrix core products.
 *   H   K x K fp32; the lower triangle is read, the full symmetric result is
 *       written in place.
 *   ws  device workspace of at least psd_project_workspace_size(K) bytes.
 * Synchronises `stream`.
 * Errors: GQ_ERR_INVALID_ARG (null pointer, K < 1, short workspace),
 *         GQ_ERR_NONFINITE (NaN/Inf in the lower triangle of H),
 *         GQ_ERR_INTERNAL (an iterate left the range the emulation needs; not
 *         expected for any input).  An all-zero H returns all zeros.
 */
int psd_project(float *H, int64_t K, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes gptq_factor needs for size K. */
size_t gptq_factor_workspace_size(int64_t K);

/*
 * gptq_factor -- the Cholesky-based inverse GPTQ sweeps with (ork-driver wiki,
 * "Exp 2026-08-18 GPTQ Int4": Cholesky-based Hessian inverse).
 * mu = mean(diag H); H_d = H + damp * mu * I (damping in units of mean(diag H),
 * hipfire-calib-data, "The fix"); U is the upper-triangular factor with
 * H_d^{-1} = U^T U.  Computed in fp64 as U = R^{-1} where H_d = R R^T with R
 * upper triangular (the Cholesky factor of the order-reversed H_d, reversed back).
 *   U     K x K fp32 row-major, written (zeros below the diagonal).
 *   H     K x K fp32, lower triangle read.    damp  >= 0 (0.01 on the pages).
 *   ws    at least gptq_factor_workspace_size(K) bytes.
 * Synchronises `stream`.
 * Errors: GQ_ERR_INVALID_ARG, GQ_ERR_NONFINITE (H lower triangle),
 *         GQ_ERR_NO_CALIBRATION (mu <= 0), GQ_ERR_NOT_PD (pivot <= 0).
 */
int gptq_factor(float *U, const float *H, int64_t K, float damp, void *ws, size_t ws_bytes,
                hipStream_t stream);

/* Workspace bytes gptq_sweep needs for an N x K weight with group size `group`. */
size_t gptq_sweep_workspace_size(int64_t N, int64_t K, int64_t group);

/*
 * gptq_sweep -- GPTQ error-feedback sweep of W under a given factor U (from
 * gptq_factor), emitting uniform symmetric int4 codes in [-8, 7] with one scale
 * absmax/7 per (row, group), so that w ~ code * scale (ork-driver wiki, "Exp
 * 2026-08-18 GPTQ Int4").  Columns are taken in natural order; a group's scale is
 * fixed at the group's first column from the group's current error-updated
 * values; code = clamp(rint(w / scale), -8, 7) with ties to even; the error
 * e = (w - code*scale) / U[i][i] is fed back into the later columns through row
 * i of U.  Updates are batched lazily over blocks of 128 columns.
 *   codes     N x K/2 bytes: column 2m in the low nibble of byte m of its row,
 *             two's complement.
 *   scales    N x (K/group) fp32.
 *   qerr_out  host pointer or NULL.  When non-NULL it receives
 *             sqrt(sum_n sum_k imp[k] (w - code*scale)^2 / sum_n sum_k imp[k] w^2)
 *             over the original W (0 when the denominator is 0) -- the qerr of the
 *             same wiki page.  Codes and scales are identical either way.
 *   W         N x K fp32, not modified.    U  K x K fp32 from gptq_factor.
 *   imp       K fp32 importance weights, or NULL for all ones.
 *   N >= 1; K even, K >= 2; 1 <= group <= 128, group divides 128 and K.
 *   ws        at least gptq_sweep_workspace_size(N, K, group) bytes.
 * Synchronises `stream`.
 * Errors: GQ_ERR_INVALID_ARG, GQ_ERR_NONFINITE (W or imp).
 */
int gptq_sweep(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *U,
               const float *imp, int64_t N, int64_t K, int64_t group, void *ws, size_t ws_bytes,
               hipStream_t stream);

/*
 * gptq_factor_f64 -- gptq_factor with U written in fp64: the same damping,
 * Cholesky and inverse (computed in fp64), without the rounding to fp32.
 *   U   K x K fp64 row-major, written (zeros below the diagonal).
 * Other arguments, workspace (gptq_factor_workspace_size), synchronisation and
 * errors as gptq_factor.  For tensors that share one Hessian at large K (for
 * callers sharing a Hessian across weights, ork-driver wiki, "Exp 2026-08-18
 * GPTQ Int4": the factor is per Hessian, the sweep per weight), with
 * gptq_sweep_f64.
 */
int gptq_factor_f64(double *U, const float *H, int64_t K, float damp, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/* Workspace bytes gptq_sweep_f64 needs (gptq_sweep's, plus N x K doubles). */
size_t gptq_sweep_f64_workspace_size(int64_t N, int64_t K, int64_t group);

/*
 * gptq_sweep_f64 -- gptq_sweep with its state in fp64: U (from
 * gptq_factor_f64), the working weights and the errors are fp64 and the block
 * updates run on the fp64 matrix cores; the rounding decisions are those of
 * gptq_sweep (the code of fl32(w) / s, ties to even).  This is the sweep
 * gptq_quantize runs above K = 8192, where an fp32 state drifts far enough from
 * an fp64 one to decide measurably many rounding ties the other way.  The
 * uniform grid with dynamic groups only.
 *   U   K x K fp64 from gptq_factor_f64 (upper triangle read).
 * Other arguments, synchronisation and errors as gptq_sweep; ws at least
 * gptq_sweep_f64_workspace_size(N, K, group) bytes.
 */
int gptq_sweep_f64(uint8_t *codes, float *scales, double *qerr_out, const float *W, const double *U,
                   const float *imp, int64_t N, int64_t K, int64_t group, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* Workspace bytes gptq_quantize needs. */
size_t gptq_quantize_workspace_size(int64_t N, int64_t K, int64_t group);

/*
 * gptq_quantize -- damping, blocked Cholesky, U, and the lazy-batch sweep in one
 * call: gptq_factor into the workspace, then gptq_sweep.  Arguments as above;
 * H is K x K fp32 (lower triangle read), damp the damping fraction (0.01).
 * Above K = 8192 the sweep keeps U (the same fp64 factor gptq_factor rounds to
 * fp32), the working weights and the errors in fp64, with its block updates on
 * the fp64 matrix cores: over rows that long an fp32 state drifts far enough
 * from an fp64 one to decide measurably many rounding ties the other way.  The
 * rounding decisions themselves are fp32 in both (the code of fl32(w) / s).
 * The workspace (gptq_quantize_workspace_size) includes the N x K doubles this
 * needs at every K.
 * Synchronises `stream`.
 */
int gptq_quantize(uint8_t *codes, float *scales, double *qerr_out, const float *W,
                  const float *H, const float *imp, int64_t N, int64_t K, int64_t group,
                  float damp, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Variants of the sweep and of the round-to-nearest pack, added as new symbols
 * that the originals forward to with flags = 0 (ork-driver wiki, "Exp 2026-08-18
 * GPTQ Int4": extend by a variant, never by changing a signature).  Flag bits:
 *   GQ_STATIC_GROUPS  every (row, group) scale is fixed before the sweep from the
 *                     original weights (as AutoGPTQ's static_groups), instead of
 *                     at the group's first column from its error-updated values.
 *                     Error feedback may then carry a value past the grid's
 *                     ends, where the code clamps.  No effect on rtn_quantize_ex,
 *                     whose scales are always the original weights'.
 *   GQ_NF4            the 16-level NF4 codebook (the 4-bit pack the same wiki's
 *                     qerr section scores beside the uniform grid) instead of the
 *                     uniform int4 grid: scale = absmax of the group, code = the
 *                     unsigned index 0..15 of the level nearest to w / scale
 *                     (a value on the midpoint of two levels takes the lower),
 *                     w ~ level[code] * scale; an all-zero group takes code 7
 *                     (level 0.0).  gq_nf4_levels gives the table.
 *   GQ_ACT_ORDER      (gptq_quantize_ex only, with GQ_STATIC_GROUPS) columns are
 *                     quantised in order of decreasing diag(H) (AutoGPTQ's
 *                     desc_act; equal entries in column order): H is permuted on
 *                     both sides and factored, and each column keeps its original
 *                     contiguous group's static scale, so codes and scales come
 *                     back in the ordinary layout (original column order).
 * Other bits are GQ_ERR_INVALID_ARG.  Codes are packed two per byte as for
 * gptq_sweep (unsigned nibbles under GQ_NF4); qerr uses the dequantised value of
 * the chosen grid.
 */
enum { GQ_STATIC_GROUPS = 1u, GQ_NF4 = 2u, GQ_ACT_ORDER = 4u };

/* The 16 NF4 levels, ascending, fp32 (QLoRA's 4-bit NormalFloat: standard normal
 * quantiles at evenly spaced probabilities, 7 below zero and 8 above, the
 * outermost at 1 - (1/32 + 1/30)/2, scaled to [-1, 1]).  levels: host, 16 floats. */
void gq_nf4_levels(float *levels);

/* gptq_sweep with flags (above); everything else as gptq_sweep, same workspace. */
int gptq_sweep_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *U,
                  const float *imp, int64_t N, int64_t K, int64_t group, uint32_t flags, void *ws,
                  size_t ws_bytes, hipStream_t stream);

/* Workspace bytes gptq_quantize_ex needs: gptq_quantize's, plus with
 * GQ_ACT_ORDER a permuted K x K Hessian, the permutation and permuted codes. */
size_t gptq_quantize_ex_workspace_size(int64_t N, int64_t K, int64_t group, uint32_t flags);

/* gptq_quantize with flags (above); ws at least
 * gptq_quantize_ex_workspace_size(N, K, group, flags) bytes. */
int gptq_quantize_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *H,
                     const float *imp, int64_t N, int64_t K, int64_t group, float damp, uint32_t flags, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Block Walsh-Hadamard rotation, the rotation GPTQ composes with (ork-driver wiki,
 * "Exp 2026-08-18 GPTQ Int4": rotate, then quantise, as in QuaRot).
 * R = blockdiag(H_b, ..., H_b) diag(signs) / sqrt(b) over the K input channels,
 * H_b the Sylvester Hadamard matrix of order b (H_1 = [1],
 * H_2m = [[H_m, H_m], [H_m, -H_m]]), b = block a power of two <= 4096 that
 * divides K, signs a K-vector of +1/-1 (fp32, device) or NULL for all +1.  R is
 * orthogonal: W' = W R^T and X' = X R^T leave W X^T unchanged, and the Hessian of
 * X' is R H R^T.  Both calls are asynchronous (argument and launch errors only).
 */
/* hadamard_rotate_rows -- A[r, :] <- A[r, :] R^T for each of `rows` rows of the
 * fp32 matrix A (row r at A + r*ld, ld >= K), in place: W or X. */
int hadamard_rotate_rows(float *A, int64_t rows, int64_t K, int64_t ld, int64_t block, const float *signs,
                         hipStream_t stream);

/* Workspace bytes hadamard_rotate_hessian needs (one K x K fp32 matrix). */
size_t hadamard_rotate_hessian_workspace_size(int64_t K);

/* hadamard_rotate_hessian -- H <- R H R^T for a full symmetric K x K fp32 H (both
 * triangles read and written), in place through the workspace. */
int hadamard_rotate_hessian(float *H, int64_t K, int64_t block, const float *signs, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* Workspace bytes rtn_quantize needs (a few KB, independent of the sizes). */
size_t rtn_quantize_workspace_size(int64_t N, int64_t K, int64_t group);

/*
 * rtn_quantize -- round-to-nearest pack of W on the same int4 grid as
 * gptq_sweep, with no error feedback: per (row, group) scale absmax/7 of the
 * original weights, code = clamp(rint(w / scale), -8, 7) with an IEEE fp32
 * division and ties to even (0 for an all-zero group), and optionally the same
 * qerr.  It is the uniform pack whose qerr a re-tiering pass ranks by, and the
 * comparator GPTQ's codes are judged against (ork-driver wiki, "Exp 2026-08-18
 * GPTQ Int4": the producer of a pack's qerr field and its uniform-weight check).
 * Codes and scales are identical whether or not qerr_out is given.
 *   codes, scales, qerr_out, W, imp, N, K, group: as for gptq_sweep (device
 *             pointers except qerr_out; codes and scales written, W and imp read).
 *   ws        at least rtn_quantize_workspace_size(N, K, group) bytes.
 * Synchronises `stream`.
 * Errors: GQ_ERR_INVALID_ARG, GQ_ERR_NONFINITE (W or imp).
 */
int rtn_quantize(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp,
                 int64_t N, int64_t K, int64_t group, void *ws, size_t ws_bytes, hipStream_t stream);

/* rtn_quantize with flags (GQ_NF4: the NF4 codebook; GQ_STATIC_GROUPS changes
 * nothing); same workspace as rtn_quantize. */
int rtn_quantize_ex(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp,
                    int64_t N, int64_t K, int64_t group, uint32_t flags, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * rtn_quantize_noalloc -- rtn_quantize_ex with no workspace argument, for
 * callers that cannot allocate device memory (code that must not call
 * hipMalloc, such as tight serving loops or harnesses that forbid it).  Its
 * status word and qerr's partial sums live in a fixed scratch array of
 * GQ_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from its
 * first use on that device until the process ends; the call allocates nothing
 * and otherwise does exactly what rtn_quantize_ex does (same kernels, codes,
 * scales and qerr).  rtn_quantize_workspace_size is at most 36.5 KiB for any
 * N, K and group, so every size rtn_quantize_ex takes fits; a size that would
 * not is refused with GQ_ERR_INVALID_ARG.  Calls on one device share its
 * scratch: calls that overlap on the same device (other streams or threads)
 * race and must be serialised by the caller.  Synchronises `stream`.
 */
#define GQ_NOALLOC_SCRATCH_BYTES 65536
int rtn_quantize_noalloc(uint8_t *codes, float *scales, double *qerr_out, const float *W, const float *imp,
                         int64_t N, int64_t K, int64_t group, uint32_t flags, hipStream_t stream);

/*
 * HFQM calibration package (.calib.hfq), the container that carries stored
 * Hessians and importance vectors (hipfire-calib-data dataset card, ".calib.hfq —
 * HFQM calibration package").  Little-endian: a 32-byte header ("HFQM", version
 * u32 = 1, arch_id u32, n_entries u32, metadata_offset u64, data_offset u64), one
 * self-delimited JSON value at metadata_offset, the index right after it
 * (n_entries u32, then per entry name_len u16, name, quant_type u8, n_dims u8,
 * shape[n_dims] u32, group_size u32, data_size u64), and the payloads
 * concatenated in index order from data_offset.  A tensor contributes
 * "<name>.hessian" (quant_type GQ_HFQM_HESSIAN: the hessian_pack_tril blob, shape
 * K x K) and "<name>.imatrix" (GQ_HFQM_F32 values, shape K).  Host code and host
 * buffers only; each call opens, reads or writes and closes the file.
 * Errors: GQ_ERR_INVALID_ARG, GQ_ERR_IO (open/read/write failure, or not a
 * well-formed package: bad magic or version, offsets, index or sizes).
 */
enum { GQ_HFQM_F32 = 0, GQ_HFQM_HESSIAN = 130 };

/*
 * hfqm_write -- write a package of n_entries entries to path (replaced if it
 * exists).  metadata_json: exactly one JSON object or array, no surrounding
 * whitespace.  Entry i: names[i] (NUL-terminated, < 65536 bytes),
 * quant_types[i], n_dims[i] <= 4, shapes[4 i .. 4 i + n_dims[i] - 1],
 * group_sizes[i], and data_sizes[i] bytes at host pointer data[i].
 */
int hfqm_write(const char *path, uint32_t arch_id, const char *metadata_json, int64_t n_entries,
               const char *const *names, const uint8_t *quant_types, const uint8_t *n_dims,
               const uint32_t *shapes, const uint32_t *group_sizes, const uint64_t *data_sizes,
               const void *const *data);

/*
 * hfqm_read_header -- arch_id, entry count, data_offset and the metadata JSON of
 * the package at path.  Any output pointer may be NULL; metadata (if not NULL)
 * receives the JSON text and a NUL in metadata_cap bytes, *metadata_len its
 * length.
 */
int hfqm_read_header(const char *path, uint32_t *arch_id, int64_t *n_entries, uint64_t *data_offset,
                     char *metadata, size_t metadata_cap, size_t *metadata_len);

/*
 * hfqm_read_entry -- index entry i (0-based): name (NUL-terminated, in name_cap
 * bytes), quant_type, n_dims, shape[4] (unused dimensions 0), group_size,
 * data_size, and the byte offset of its payload in the file.  Any output pointer
 * may be NULL.
 */
int hfqm_read_entry(const char *path, int64_t i, char *name, size_t name_cap, uint8_t *quant_type,
                    uint8_t *n_dims, uint32_t *shape, uint32_t *group_size, uint64_t *data_size,
                    uint64_t *offset);

/* hfqm_read_payload -- entry i's payload into dst (a host buffer of dst_bytes >= its data_size). */
int hfqm_read_payload(const char *path, int64_t i, void *dst, size_t dst_bytes);

/*
 * ---------------------------------------------------------------------------
 * Testing and profiling controls.  Not part of the computation's contract:
 * they change how later calls on the same host thread run (which product kind
 * psd_project uses, whether it times its launches), never what a correct
 * result is.  Each setting is thread-local, starts at its default on every
 * thread, and stays until changed.
 * ---------------------------------------------------------------------------
 */

/* Per-kernel timing of psd_project, for profiling.  gq_set_timing(1) makes
 * later psd_project calls on this host thread bracket each launch of their
 * product kernel with HIP events on the caller's stream; psd_project_last_timing
 * then reports, for the last such call on this thread, the number of product
 * launches, their summed duration in ms (*product_ms), and the name of that
 * kernel (static string).  Returns GQ_ERR_INVALID_ARG if no timed call was
 * made.  Timing is off by default and costs two event records per launch. */
void gq_set_timing(int on);
int psd_project_last_timing(int *launches, double *product_ms, const char **kernel);

/* Kind of the symmetric products inside psd_project, for tests and comparisons.
 * GQ_PSD_AUTO (default): emulated in integers on the int8 matrix cores for
 * K < 65536, fp64 matrix-core products above.  GQ_PSD_F64: fp64 matrix-core
 * products at every K.  Applies to later psd_project calls on this host thread;
 * psd_project_workspace_size covers both kinds.  Returns GQ_ERR_INVALID_ARG for
 * any other value (the setting is then unchanged). */
enum { GQ_PSD_AUTO = 0, GQ_PSD_F64 = 1 };
int gq_set_psd_products(int kind);

/* State of gptq_quantize's sweep for the plain grid (flags 0), for tests and
 * comparisons.  GQ_SWEEP_AUTO (default): fp64 above K = 8192, fp32 up to it.
 * GQ_SWEEP_F32 / GQ_SWEEP_F64: that state at every K.  The variants (any flag
 * set) and gptq_sweep always sweep in fp32.  Applies to later gptq_quantize and
 * gptq_quantize_ex calls on this host thread; the workspace size covers both.
 * Returns GQ_ERR_INVALID_ARG for any other value (the setting is then
 * unchanged). */
enum { GQ_SWEEP_AUTO = 0, GQ_SWEEP_F32 = 1, GQ_SWEEP_F64 = 2 };
int gq_set_sweep_state(int kind);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
