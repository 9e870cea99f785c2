// gemm_tn.hip -- matrix-core GEMM C = alpha * A^T B + beta * Cin for the dense
// contractions of the path, with both operands "k-major" (row k of A holds a run
// of output rows, row k of B a run of output columns).
//
// Every contraction of the path has that shape without any transposition:
//   * the Gram matrix X^T X (rows of X are tokens),
//   * products of symmetric matrices X Y = X^T Y (the sign iteration),
//   * the upper Cholesky trailing update R^T R over a panel's rows,
//   * the triangular-inverse updates, and
//   * the GPTQ lazy-block update E U[blk, :] with E stored transposed.
// So operands stream from HBM with contiguous 16-byte loads straight into an LDS
// layout [k][m] from which each MFMA lane reads its element at a fixed k row:
// a whole wave reads contiguous LDS words, free of bank conflicts.
//
// Tiles are 128 x 128 per 256-thread workgroup (2 x 2 waves of 64 x 64), k in
// stages of 16 rows, LDS double-buffered so the global loads of stage k+1 are in
// flight while the matrix cores work on stage k.
//   fp32: v_mfma_f32_32x32x2f32, 2 x 2 blocks of 32 x 32 per wave.
//   fp64: v_mfma_f64_16x16x4f64, 4 x 4 blocks of 16 x 16 per wave.
#include <algorithm>

#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16, NT = 256;

template <typename T> struct Mfma;

template <> struct Mfma<float> {
    static constexpr int BLK = 32;          // output block edge of one instruction
    static constexpr int NB = 64 / BLK;     // blocks per wave edge
    static constexpr int KSTEP = 2;         // k consumed per instruction
    static constexpr int LPK = 32;          // lanes per k row: lane -> (k = l / 32, m = l % 32)
    static constexpr int NACC = 16;
    typedef f32x16 acc_t;
    __device__ static acc_t mma(float a, float b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // accumulator element r of lane -> (row, col) inside the 32 x 32 block
    __device__ static int row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
    __device__ static int col(int lane, int) { return lane & 31; }
};

template <> struct Mfma<double> {
    static constexpr int BLK = 16;
    static constexpr int NB = 64 / BLK;
    static constexpr int KSTEP = 4;
    static constexpr int LPK = 16;          // lane -> (k = l / 16, m = l % 16)
    static constexpr int NACC = 4;
    typedef f64x4 acc_t;
    __device__ static acc_t mma(double a, double b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // the fp64 instruction interleaves rows across lane groups: element r of
    // lane l is row l/16 + 4 r (unlike the 4 (l/16) + r of the fp32 16x16 shapes)
    __device__ static int row(int lane, int r) { return (lane >> 4) + 4 * r; }
    __device__ static int col(int lane, int) { return lane & 15; }
};

__device__ inline double ipow(double x, int p)
{
    double r = 1.0;
    for (int i = 0; i < p; ++i) r *= x;
    return r;
}

// Tile order.  Workgroup w runs on XCD w % 8 (round-robin dispatch), and each
// XCD has its own L2.  The j-th workgroup of XCD x is given logical tile
// base_x + j, so each XCD walks a contiguous stretch of the logical order; the
// logical order visits tiles in groups of kGroup tile rows, column by column, so
// the workgroups resident on one XCD at a time cover a compact block of tiles
// and read the same A and B panels through its L2.
constexpr int kXcd = 8;
constexpr int64_t kGroup = 8;

__device__ inline int64_t xcd_logical(int64_t w, int64_t n)
{
    const int64_t x = w % kXcd, j = w / kXcd;
    int64_t base = 0;
    for (int64_t y = 0; y < x; ++y) base += (n - y + kXcd - 1) / kXcd;
    return base + j;
}

// Rectangular tm x tn grid, grouped by kGroup tile rows.
__device__ inline void rect_tile(int64_t l, int64_t tm, int64_t tn, int64_t &ti, int64_t &tj)
{
    const int64_t per = kGroup * tn;
    const int64_t g = l / per, r = l % per;
    const int64_t rows = (tm - g * kGroup) < kGroup ? (tm - g * kGroup) : kGroup;
    tj = r / rows;
    ti = g * kGroup + r % rows;
}

// Lower triangle (ti >= tj) of an nt x nt grid, grouped by kGroup tile rows:
// group g holds rows [g*G, g*G+G); within it, column tj lists rows max(tj, g*G)..
// All full groups before g hold sum over their rows of (row+1) tiles.
__device__ inline void lower_tile(int64_t l, int64_t nt, int64_t &ti, int64_t &tj)
{
    int64_t g = 0, start = 0;
    for (;;) {
        const int64_t r0 = g * kGroup;
        const int64_t r1 = (r0 + kGroup < nt) ? r0 + kGroup : nt;
        const int64_t cnt = (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2;   // tiles in rows [r0, r1)
        if (l < start + cnt) {
            int64_t off = l - start;
            // columns 0 .. r0-1 have (r1 - r0) rows each
            const int64_t full = r0 * (r1 - r0);
            if (off < full) {
                tj = off / (r1 - r0);
                ti = r0 + off % (r1 - r0);
            } else {
                off -= full;           // columns r0 .. r1-1: column c has rows c .. r1-1
                int64_t c = r0;
                while (off >= r1 - c) { off -= r1 - c; ++c; }
                tj = c;
                ti = c + off;
            }
            return;
        }
        start += cnt;
        ++g;
    }
}

// Operand loading, the MFMA main loop over a range of k stages, and the
// epilogue of one 128 x 128 tile, shared by the tile-per-workgroup kernel and
// the stream-K kernels below.
template <typename T> struct Tile {
    using MF = Mfma<T>;
    static constexpr int V = 16 / (int)sizeof(T);       // elements per 16-byte vector
    static constexpr int LDP = BM + V;                   // padded LDS row (elements)
    static constexpr int VPR = BM / V;                   // vectors per tile row
    // k rows per stage: 32 for fp32 (half the barriers per matrix instruction;
    // two workgroups still share a CU's LDS), 16 for fp64 (the DMA ring's layout)
    static constexpr int KB = sizeof(T) == 4 ? 2 * BK : BK;
    static constexpr int NV = KB * VPR / NT;             // vectors per thread per operand
    typedef T vec_t __attribute__((ext_vector_type(V)));
    typedef typename MF::acc_t acc_t;
    struct Smem {
        T As[2][KB][LDP];
        T Bs[2][KB][LDP];
    };

    // acc = sum over k stages [s0, s1) of A[k][i0 + i] * B[k][j0 + j].
    // Interior stages load whole 16-byte vectors unconditionally; edge stages
    // load element by element from clamped (always valid) addresses and zero the
    // out-of-range elements with a select, so no lane ever branches.
    template <int DP = (sizeof(T) == 4 ? 2 : 1)>
    __device__ static void mainloop(const GemmDesc &d, int64_t i0, int64_t j0, int64_t s0, int64_t s1,
                                    int vecA, int vecB, Smem &sm, acc_t (&acc)[MF::NB][MF::NB])
    {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wr = wave >> 1, wc = wave & 1;
        const T *A = (const T *)d.A;
        const T *B = (const T *)d.B;
        const bool full_i = vecA && (i0 + BM <= d.M);
        const bool full_j = vecB && (j0 + BN <= d.N);
#pragma unroll
        for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
                for (int r = 0; r < MF::NACC; ++r) acc[bi][bj][r] = (T)0;
        if (s1 <= s0) return;

        // Global loads go through registers: fp32 keeps two stages in flight
        // (a stage of its 64-cycle instructions is shorter than a load under
        // load), fp64 one.
        constexpr int D = DP;
        vec_t ra[D][NV], rb[D][NV];
        auto gload = [&](int64_t kb, int sl) {
            const bool full_k = kb + KB <= d.Kd;
            if (full_i && full_k) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int lin = tid + NT * v;
                    const int kr = lin / VPR, cc = (lin % VPR) * V;
                    ra[sl][v] = *(const vec_t *)(A + (kb + kr) * d.lda + i0 + cc);
                }
            } else {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int lin = tid + NT * v;
                    const int kr = lin / VPR, cc = (lin % VPR) * V;
                    const int64_t k = kb + kr;
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const bool ok = k < d.Kd && i0 + cc + e < d.M;
                        const T x = A[ok ? k * d.lda + i0 + cc + e : 0];
                        ra[sl][v][e] = ok ? x : (T)0;
                    }
                }
            }
            if (full_j && full_k) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int lin = tid + NT * v;
                    const int kr = lin / VPR, cc = (lin % VPR) * V;
                    rb[sl][v] = *(const vec_t *)(B + (kb + kr) * d.ldb + j0 + cc);
                }
            } else {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int lin = tid + NT * v;
                    const int kr = lin / VPR, cc = (lin % VPR) * V;
                    const int64_t k = kb + kr;
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const bool ok = k < d.Kd && j0 + cc + e < d.N;
                        const T x = B[ok ? k * d.ldb + j0 + cc + e : 0];
                        rb[sl][v][e] = ok ? x : (T)0;
                    }
                }
            }
        };
        auto sstore = [&](int buf, int sl) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int lin = tid + NT * v;
                const int kr = lin / VPR, cc = (lin % VPR) * V;
                *(vec_t *)&sm.As[buf][kr][cc] = ra[sl][v];
                *(vec_t *)&sm.Bs[buf][kr][cc] = rb[sl][v];
            }
        };
        auto compute = [&](int buf) {
            const int m = lane % MF::LPK;
#pragma unroll
            for (int kk = 0; kk < KB; kk += MF::KSTEP) {
                const int kr = kk + lane / MF::LPK;
                T a[MF::NB], b[MF::NB];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi) a[bi] = sm.As[buf][kr][wr * 64 + bi * MF::BLK + m];
#pragma unroll
                for (int bj = 0; bj < MF::NB; ++bj) b[bj] = sm.Bs[buf][kr][wc * 64 + bj * MF::BLK + m];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < MF::NB; ++bj) acc[bi][bj] = MF::mma(a[bi], b[bj], acc[bi][bj]);
            }
        };

        gload(s0 * KB, 0);
        sstore(0, 0);
        if constexpr (D == 2) {
            if (s0 + 1 < s1) gload((s0 + 1) * KB, 1);
        }
        __syncthreads();
        if constexpr (D == 2) {
            // stage kt sits in LDS buffer (kt - s0) & 1; stage kt + 1 in register
            // slot (kt - s0 + 1) & 1, and stage kt + 2 is loaded into the other
            int64_t kt = s0;
            auto iter = [&](auto SL) {
                constexpr int sl = decltype(SL)::value;        // (kt - s0) & 1
                if (kt + 2 < s1) gload((kt + 2) * KB, sl);
                compute(sl);
                if (kt + 1 < s1) sstore(sl ^ 1, sl ^ 1);
                __syncthreads();
                ++kt;
            };
            while (kt + 1 < s1) {
                iter(std::integral_constant<int, 0>{});
                iter(std::integral_constant<int, 1>{});
            }
            if (kt < s1) iter(std::integral_constant<int, 0>{});
        } else {
            for (int64_t kt = s0; kt < s1; ++kt) {
                const int buf = (int)((kt - s0) & 1);
                if (kt + 1 < s1) gload((kt + 1) * KB, 0);
                compute(buf);
                if (kt + 1 < s1) sstore(buf ^ 1, 0);
                __syncthreads();
            }
        }
    }

    // The same sum with the operands copied by the DMA path (global_load_lds:
    // each wave instruction lands 64 x 16 bytes, one 128-element row, straight
    // in LDS, with no registers held for it), in sub-stages of SUB rows through
    // a ring of RING buffers that keeps three sub-stages in flight.  It uses the
    // same LDS as the two 16-row buffers of mainloop, so two workgroups still
    // share a CU.  Preconditions, checked by the launcher: every row of A and B
    // starts 16-byte aligned, M and N are even (so the last 16-byte column pair
    // of a row exists: columns past M or N read their clamped neighbours, whose
    // products land only in discarded outputs) and Kd is a multiple of 16 (no
    // partial k rows, which would have to be zero).  Stage indices count 16-row
    // stages, as in mainloop.
    static constexpr int SUB = 8, RING = 4;
    // One DMA row copy: each lane's 16 bytes at gptr land at LDS byte address
    // lds + 16 * lane.  Issued from asm so that the compiler, which cannot tell
    // the ring's slots apart, adds no waits of its own; every wait is explicit
    // below.  No register is written by the instruction.
    __device__ static void dma_row(const T *gptr, const T *lds)
    {
        typedef __attribute__((address_space(3))) const void lds_cvoid;
        const unsigned addr = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_cvoid *)lds);
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(gptr), "s"(addr)
                     : "memory", "m0");
    }
    __device__ static void mainloop_dma(const GemmDesc &d, int64_t i0, int64_t j0, int64_t s0, int64_t s1,
                                        Smem &sm, acc_t (&acc)[MF::NB][MF::NB])
    {
        static_assert(sizeof(T) == 8 && RING * SUB == 2 * BK, "the DMA ring is laid out for fp64 in Smem");
        T(*As)[LDP] = &sm.As[0][0];                     // RING * SUB rows of the same storage
        T(*Bs)[LDP] = &sm.Bs[0][0];
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
        for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
                for (int r = 0; r < MF::NACC; ++r) acc[bi][bj][r] = (T)0;
        if (s1 <= s0) return;
        const int64_t q0 = 2 * s0, q1 = 2 * s1;
        // this wave copies rows 2 wave and 2 wave + 1 of each sub-stage of A and B
        const int64_t ca = (i0 + 2 * lane) < d.M - 2 ? i0 + 2 * lane : d.M - 2;
        const int64_t cb = (j0 + 2 * lane) < d.N - 2 ? j0 + 2 * lane : d.N - 2;
        const T *pa = (const T *)d.A + ca + (int64_t)(2 * wave) * d.lda;
        const T *pb = (const T *)d.B + cb + (int64_t)(2 * wave) * d.ldb;
        auto issue = [&](int64_t q, int slot) {
            const int64_t kb = q * SUB;
            const T *la = As[slot * SUB + 2 * wave];
            const T *lb = Bs[slot * SUB + 2 * wave];
            dma_row(pa + kb * d.lda, la);
            dma_row(pa + (kb + 1) * d.lda, la + LDP);
            dma_row(pb + kb * d.ldb, lb);
            dma_row(pb + (kb + 1) * d.ldb, lb + LDP);
        };
        // Waits are explicit: vmcnt(n) = at most n of this wave's vector memory
        // operations outstanding (they complete in order), with lgkmcnt(0) so
        // that this wave's LDS reads are done before the barrier frees their
        // buffer.  s_waitcnt immediates on this target: vmcnt in bits 3:0,
        // expcnt 6:4 (7 = no wait), lgkmcnt 11:8.
        __builtin_amdgcn_s_waitcnt(0x0070);             // stores of the previous tile, if any
        __builtin_amdgcn_s_barrier();                   // every wave is done with the ring
        asm volatile("" ::: "memory");
        issue(q0, 0);
        if (q0 + 1 < q1) issue(q0 + 1, 1);
        if (q0 + 2 < q1) issue(q0 + 2, 2);
        const int m = lane % MF::LPK;
        for (int64_t q = q0; q < q1; ++q) {
            const int slot = (int)((q - q0) & (RING - 1));
            const int64_t later = (q1 - 1 - q) < 2 ? (q1 - 1 - q) : 2;   // sub-stages issued after q
            if (later == 2) __builtin_amdgcn_s_waitcnt(0x0078);
            else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0074);
            else __builtin_amdgcn_s_waitcnt(0x0070);
            __builtin_amdgcn_s_barrier();                // sub-stage q is in LDS for every wave,
            asm volatile("" ::: "memory");               // and slot q - 1 is free
            if (q + 3 < q1) issue(q + 3, (slot + 3) & (RING - 1));
            const T(*Aq)[LDP] = As + slot * SUB;
            const T(*Bq)[LDP] = Bs + slot * SUB;
#pragma unroll
            for (int kk = 0; kk < SUB; kk += MF::KSTEP) {
                const int kr = kk + lane / MF::LPK;
                T a[MF::NB], b[MF::NB];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi) a[bi] = Aq[kr][wr * 64 + bi * MF::BLK + m];
#pragma unroll
                for (int bj = 0; bj < MF::NB; ++bj) b[bj] = Bq[kr][wc * 64 + bj * MF::BLK + m];
#pragma unroll
                for (int bi = 0; bi < MF::NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < MF::NB; ++bj) acc[bi][bj] = MF::mma(a[bi], b[bj], acc[bi][bj]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();                   // the ring may be refilled by the next tile
        asm volatile("" ::: "memory");
    }

    template <typename OutT>
    __device__ static void epilogue(const GemmDesc &d, int64_t i0, int64_t j0, const acc_t (&acc)[MF::NB][MF::NB])
    {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wr = wave >> 1, wc = wave & 1;
        double alpha = d.alpha, beta = d.beta;
        if (d.alpha_dev) alpha *= ipow(*d.alpha_dev, d.alpha_pow);
        if (d.beta_dev) beta *= ipow(*d.beta_dev, d.beta_pow);
        OutT *out = (OutT *)d.out;
        OutT *out_t = (OutT *)d.out_t;
        const T *cin = (const T *)d.cin;
        // One row of blocks at a time (32 fp32 or 16 fp64 values per lane): its
        // cin values are all loaded, from clamped addresses, before any is used,
        // so the tile waits on memory once per block row rather than once per
        // element.
#pragma unroll
        for (int bi = 0; bi < MF::NB; ++bi) {
            T c[MF::NB][MF::NACC];
            if (beta != 0.0) {
#pragma unroll
                for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
                    for (int r = 0; r < MF::NACC; ++r) {
                        const int64_t gi = i0 + wr * 64 + bi * MF::BLK + MF::row(lane, r);
                        const int64_t gj = j0 + wc * 64 + bj * MF::BLK + MF::col(lane, r);
                        const bool in = gi < d.M && gj < d.N;
                        c[bj][r] = cin[in ? gi * d.ldc + gj : 0];
                    }
            }
#pragma unroll
            for (int bj = 0; bj < MF::NB; ++bj)
#pragma unroll
                for (int r = 0; r < MF::NACC; ++r) {
                    const int64_t gi = i0 + wr * 64 + bi * MF::BLK + MF::row(lane, r);
                    const int64_t gj = j0 + wc * 64 + bj * MF::BLK + MF::col(lane, r);
                    if (gi >= d.M || gj >= d.N) continue;
                    if (d.tri == 1 && gi < gj) continue;
                    if (d.tri == 2 && gi > gj) continue;
                    double v = alpha * (double)acc[bi][bj][r];
                    if (beta != 0.0) v += beta * (double)c[bj][r];
                    out[gi * d.ldo + gj] = (OutT)v;
                    if (out_t) out_t[gj * d.ldo + gi] = (OutT)v;
                }
        }
    }
};

__device__ inline void tile_coords(const GemmDesc &d, int64_t l, int64_t tiles_m, int64_t tiles_n,
                                   int64_t &i0, int64_t &j0)
{
    int64_t ti, tj;
    if (d.mode == TILE_RECT) {
        rect_tile(l, tiles_m, tiles_n, ti, tj);
    } else {
        lower_tile(l, tiles_m, ti, tj);
        if (d.mode == TILE_UPPER) { int64_t t = ti; ti = tj; tj = t; }
    }
    i0 = ti * BM;
    j0 = tj * BN;
}

// Two waves per SIMD: without the hint the fp64 instance keeps its 64-double
// accumulator in AGPRs next to 238 VGPRs, one wave per SIMD, and every stage
// stalls on its own loads; with it, 250 VGPRs and no AGPR copies.
template <typename T, typename OutT>
__global__ __launch_bounds__(NT, 2) void gemm_tn_kernel(GemmDesc d, int64_t tiles_m, int64_t tiles_n, int vecA,
                                                       int vecB)
{
    using TL = Tile<T>;
    __shared__ __attribute__((aligned(16))) typename TL::Smem sm;
    int64_t i0, j0;
    tile_coords(d, xcd_logical(blockIdx.x, gridDim.x), tiles_m, tiles_n, i0, j0);
    typename TL::acc_t acc[TL::MF::NB][TL::MF::NB];
    TL::mainloop(d, i0, j0, 0, (d.Kd + TL::KB - 1) / TL::KB, vecA, vecB, sm, acc);
    TL::template epilogue<OutT>(d, i0, j0, acc);
}

// fp64 grids of at most kSmallTiles tiles (the factor's block-row updates, which
// lie on its critical chain, and the smallest trailing and inverse updates):
// occupancy is moot there, so one wave per SIMD with the loads two stages ahead,
// as the fp32 ones are, and each stage's load latency hides behind two stages
// of matrix work.  Larger grids keep two waves per SIMD.
constexpr int64_t kSmallTiles = 64;
template <typename OutT>
__global__ __launch_bounds__(NT, 1) void gemm_tn_small_f64_kernel(GemmDesc d, int64_t tiles_m, int64_t tiles_n,
                                                                  int vecA, int vecB)
{
    using TL = Tile<double>;
    __shared__ __attribute__((aligned(16))) typename TL::Smem sm;
    int64_t i0, j0;
    tile_coords(d, xcd_logical(blockIdx.x, gridDim.x), tiles_m, tiles_n, i0, j0);
    typename TL::acc_t acc[TL::MF::NB][TL::MF::NB];
    TL::template mainloop<2>(d, i0, j0, 0, (d.Kd + TL::KB - 1) / TL::KB, vecA, vecB, sm, acc);
    TL::template epilogue<OutT>(d, i0, j0, acc);
}

// Stream-K with a data-parallel head: a persistent grid of exactly the
// resident workgroups.  The first dp_tiles tiles (whole waves) go one per
// worker per round in the grouped order, so the workgroups resident on one XCD
// share panels through its L2 as in the plain kernel.  The (tile, k-stage)
// iteration space of the remaining tiles (one to two waves' worth) is cut into
// equal contiguous shares, one per worker, so the last waves keep every CU
// equally busy whatever the tile count.  A worker finishes the tiles its share
// covers entirely.  A tile that a share boundary cuts (each share spans at
// least one tile, so a tile has at most one cut) has a head part, which ends
// the share of the worker before the boundary, and a tail part, which begins
// the share of the worker after it.  Whichever side finishes second adds the
// other's partial accumulator to its own and runs the epilogue; a counter per
// boundary decides which side that is, so no workgroup ever waits for another.
// The sum is head + tail whichever side forms it (floating-point addition is
// commutative), so results do not depend on timing.
struct StreamK {
    int64_t tiles_m, tiles_n, ntiles, nstage, workers, dp_tiles;
    // first iteration of worker w's share; w = workers gives the end
    __device__ int64_t share_begin(int64_t w) const
    {
        return dp_tiles * nstage + w * ((ntiles - dp_tiles) * nstage) / workers;
    }
};

template <typename T, typename OutT, bool DMA>
__global__ __launch_bounds__(NT, 2) void gemm_tn_streamk_kernel(GemmDesc d, StreamK k, int vecA, int vecB,
                                                               T *partials, unsigned *flags)
{
    using TL = Tile<T>;
    __shared__ __attribute__((aligned(16))) typename TL::Smem sm;
    const int64_t w = xcd_logical(blockIdx.x, gridDim.x);
    typename TL::acc_t acc[TL::MF::NB][TL::MF::NB];
    int64_t dp = w;                                     // next data-parallel tile
    int64_t it = k.share_begin(w);                      // next stream-K iteration
    const int64_t end = k.share_begin(w + 1);
    // one loop for both phases keeps a single copy of the main loop and epilogue
    for (;;) {
        int64_t tile, s0, s1;
        if (dp < k.dp_tiles) {
            tile = dp;
            s0 = 0;
            s1 = k.nstage;
            dp += k.workers;
        } else if (it < end) {
            tile = it / k.nstage;
            s0 = it - tile * k.nstage;
            s1 = (end - tile * k.nstage) < k.nstage ? (end - tile * k.nstage) : k.nstage;
            it = tile * k.nstage + s1;
        } else {
            break;
        }
        int64_t i0, j0;
        tile_coords(d, tile, k.tiles_m, k.tiles_n, i0, j0);
        if constexpr (DMA)
            TL::mainloop_dma(d, i0, j0, s0, s1, sm, acc);
        else
            TL::mainloop(d, i0, j0, s0, s1, vecA, vecB, sm, acc);
        bool epi = (s0 == 0 && s1 == k.nstage);
        unsigned *flag = nullptr;
        if (!epi) {
            // boundary b cuts this tile: the head part ends at b (this worker is
            // b - 1), the tail part starts at b (this worker is b)
            const bool head = (s0 == 0);
            const int64_t b = head ? w + 1 : w;
            flag = flags + (b - 1);
            T *mine = partials + ((b - 1) * 2 + (head ? 0 : 1)) * (int64_t)(BM * BN);
            const T *other = partials + ((b - 1) * 2 + (head ? 1 : 0)) * (int64_t)(BM * BN);
            const int tid = threadIdx.x;
            __shared__ unsigned s_prev;
            // The head part usually finishes last (it ends a share); if the tail
            // has already posted, skip storing the head part.
            if (tid == 0)
                s_prev = head ? __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            __syncthreads();
            epi = (s_prev == 1u);
            __syncthreads();
            if (!epi) {
#pragma unroll
                for (int bi = 0; bi < TL::MF::NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < TL::MF::NB; ++bj)
#pragma unroll
                        for (int r = 0; r < TL::MF::NACC; ++r)
                            mine[((bi * TL::MF::NB + bj) * TL::MF::NACC + r) * NT + tid] = acc[bi][bj][r];
                __threadfence();                        // publish the partial device-wide
                __syncthreads();
                if (tid == 0) s_prev = atomicAdd(flag, 1u);
                __syncthreads();
                epi = (s_prev == 1u);
                __syncthreads();
            }
            if (epi) {
                __threadfence();                        // see the other side's partial
#pragma unroll
                for (int bi = 0; bi < TL::MF::NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < TL::MF::NB; ++bj)
#pragma unroll
                        for (int r = 0; r < TL::MF::NACC; ++r)
                            acc[bi][bj][r] += other[((bi * TL::MF::NB + bj) * TL::MF::NACC + r) * NT + tid];
            }
        }
        if (epi) {
            TL::template epilogue<OutT>(d, i0, j0, acc);
            // the side that finished a split tile re-arms its counter
            if (flag && threadIdx.x == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <typename T, typename OutT>
hipError_t launch(const GemmDesc &d, hipStream_t s)
{
    if (d.M <= 0 || d.N <= 0) return hipSuccess;
    constexpr int V = 16 / (int)sizeof(T);
    const int64_t tm = (d.M + BM - 1) / BM, tn = (d.N + BN - 1) / BN;
    int64_t ntiles;
    if (d.mode == TILE_RECT) {
        ntiles = tm * tn;
    } else {
        if (d.M != d.N) return hipErrorInvalidValue;
        ntiles = tm * (tm + 1) / 2;
    }
    const int vecA = (d.lda % V == 0) && (((uintptr_t)d.A & 15) == 0);
    const int vecB = (d.ldb % V == 0) && (((uintptr_t)d.B & 15) == 0);
    if constexpr (sizeof(T) == 8) {
        if (ntiles <= kSmallTiles) {
            hipLaunchKernelGGL((gemm_tn_small_f64_kernel<OutT>), dim3((unsigned)ntiles), dim3(NT), 0, s, d, tm, tn,
                               vecA, vecB);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_tn_kernel<T, OutT>), dim3((unsigned)ntiles), dim3(NT), 0, s, d, tm, tn,
                       vecA, vecB);
    return hipGetLastError();
}

int resident_workers()
{
    static int w = 0;
    if (w == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        w = 2 * cus;                                    // two workgroups per CU (occupancy hint)
    }
    return w;
}

template <typename T, typename OutT>
hipError_t launch_streamk(const GemmDesc &d, void *partials, unsigned *flags, hipStream_t s)
{
    if (d.M <= 0 || d.N <= 0) return hipSuccess;
    constexpr int V = 16 / (int)sizeof(T);
    if (d.mode != TILE_RECT && d.M != d.N) return hipErrorInvalidValue;
    StreamK k;
    k.tiles_m = (d.M + BM - 1) / BM;
    k.tiles_n = (d.N + BN - 1) / BN;
    k.ntiles = (d.mode == TILE_RECT) ? k.tiles_m * k.tiles_n : k.tiles_m * (k.tiles_m + 1) / 2;
    k.nstage = (d.Kd + BK - 1) / BK;
    k.workers = std::min<int64_t>(resident_workers(), kStreamKMaxWorkers);
    if (!partials || !flags || k.ntiles < k.workers || k.nstage < 1) return launch<T, OutT>(d, s);
    // all but the last one to two waves run data-parallel
    k.dp_tiles = (k.ntiles / k.workers - 1) * k.workers;
    const int vecA = (d.lda % V == 0) && (((uintptr_t)d.A & 15) == 0);
    const int vecB = (d.ldb % V == 0) && (((uintptr_t)d.B & 15) == 0);
    const bool dma = (d.Kd % BK == 0) && (d.M % 2 == 0) && (d.N % 2 == 0) && (d.lda % 2 == 0) &&
                     (d.ldb % 2 == 0) && (((uintptr_t)d.A & 15) == 0) && (((uintptr_t)d.B & 15) == 0);
    if (dma)
        hipLaunchKernelGGL((gemm_tn_streamk_kernel<T, OutT, true>), dim3((unsigned)k.workers), dim3(NT), 0, s, d, k,
                           vecA, vecB, (T *)partials, flags);
    else
        hipLaunchKernelGGL((gemm_tn_streamk_kernel<T, OutT, false>), dim3((unsigned)k.workers), dim3(NT), 0, s, d,
                           k, vecA, vecB, (T *)partials, flags);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_tn_f32(const GemmDesc &d, hipStream_t s) { return launch<float, float>(d, s); }
hipError_t gemm_tn_f64(const GemmDesc &d, hipStream_t s) { return launch<double, double>(d, s); }
hipError_t gemm_tn_f64_out_f32(const GemmDesc &d, hipStream_t s) { return launch<double, float>(d, s); }
hipError_t gemm_tn_f64_streamk(const GemmDesc &d, void *partials, unsigned *flags, hipStream_t s)
{
    return launch_streamk<double, double>(d, partials, flags, s);
}
hipError_t gemm_tn_f64_out_f32_streamk(const GemmDesc &d, void *partials, unsigned *flags, hipStream_t s)
{
    return launch_streamk<double, float>(d, partials, flags, s);
}

}  // namespace gq
