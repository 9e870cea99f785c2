// gram_bf16.hip -- H_lower += X^T X for bf16 activations on the bf16 matrix cores.
//
// The calibration Hessian is the Gram matrix of the activations, summed over
// tokens, and chunk sums add (hipfire-calib-data, "Hessian storage"; AtomicChat
// GGUF page, "The importance matrix").  Products of two bf16 values are exact
// in fp32; each launch accumulates its chunk in fp32 registers from zero and adds
// the result to H once, so streaming many chunks rounds once per chunk and the
// result does not depend on scheduling.
//
// One workgroup per lower 256 x 256 tile (tile order as in the int8 product:
// XCD-contiguous, grouped by tile rows), 8 waves of 64 x 128 (4 x 2), each 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16.  The instruction computes X Y^T for
// 32-row panels X and Y of 16 k: lane l feeds k = 8 (l / 32) + 0..7 of row
// l % 32 of each, and result e of lane l is (X Y^T)[8 (e/4) + 4 (l/32) + e%4][l % 32].
//
// X is token-major, the instruction wants 8 consecutive tokens of one channel
// per lane: the transpose happens on the way into LDS.  A stage is 32 tokens;
// each of the 256 loader threads of a panel loads a 4-token x 8-channel patch
// (four 16-byte loads, three stages ahead into registers) and stores 8 words of
// 4 tokens, one per channel.  A panel in LDS is 256 rows of 64 bytes (32
// tokens); channel rho lives in physical row 32 (rho % 8) + rho / 8 and its
// 16-byte token chunk c at position c ^ (rho % 4) ^ (rho / 64 % 4).  A wave
// loads 2 token rows x 512 bytes per instruction (X rows are far apart, so
// wide contiguous segments keep many L2 channels busy); with that placement its
// 8-byte stores of one channel index spread over all banks, and so do the
// 16-byte matrix-operand reads of 32 consecutive channels.
#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 256;                    // tile edge (channels)
constexpr int GBT = 32;                     // tokens per stage
constexpr int GNT = 512;                    // threads
constexpr int kPanelBytes = GBM * GBT * 2;  // 16 KiB
// dynamic LDS: two slots of the A and B panels
constexpr size_t kGramLds = (size_t)4 * kPanelBytes;
// lgkmcnt(0) only: loads in flight to registers are not waited for
constexpr int kWaitLgkm0 = 0xC07F;

// VEC: K % 8 == 0 and X 16-byte aligned, so that every 8-channel octet is
// wholly inside or wholly outside [0, K) and loads as one 16-byte word.
template <bool VEC>
__global__ __launch_bounds__(GNT, 1) void gram_bf16_kernel(float *__restrict__ H,
                                                           const uint16_t *__restrict__ X,
                                                           int64_t T, int64_t K)
{
    extern __shared__ __attribute__((aligned(1024))) int8_t g_lds[];
    const int64_t nt = (K + GBM - 1) / GBM;
    int64_t ti, tj;
    lower_tile_grouped(xcd_order(blockIdx.x, gridDim.x), nt, ti, tj);
    const int64_t i0 = ti * GBM, j0 = tj * GBM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    // loader role: threads 0..255 -> panel A (channels i0..), 256..511 -> panel B
    // (channels j0.., which on a diagonal tile are A's again); channels
    // 8 o .. 8 o + 7, tokens 4 q .. 4 q + 3 of each stage
    const int panel = tid >> 8, u = tid & 255;
    const int o = u & 31, q = u >> 5;        // a wave instruction: 2 token rows x 512 bytes
    const int64_t cbase = (panel ? j0 : i0) + 8 * o;
    // byte offset of this thread's patch from the start of its stage's first
    // token row (below 2^32 for K < 2^24), and whether its octet is in range
    const unsigned voff = (unsigned)((4 * q * K + cbase) * 2);
    const bool c_in = cbase < K;
    // Stages past T load zeros: the stage count is rounded up to a multiple of
    // 6 (the pipeline's period), so that the pipeline below needs no run-time cases.
    const int64_t nk = ((T + GBT - 1) / GBT + 5) / 6 * 6 > 0 ? ((T + GBT - 1) / GBT + 5) / 6 * 6 : 6;

    u32x4 g[3][4];
    auto gload = [&](auto P, int64_t kt) {
        constexpr int p = decltype(P)::value;
        const int64_t t0 = kt * GBT + 4 * q;
        if constexpr (VEC) {
            // Address = uniform row base (clamped into X) + per-thread byte
            // offset; out-of-range rows read the first 8 channels of a valid row
            // and lstore replaces them by zeros (a select here would wait for
            // the load at once).
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = kt * GBT + r < T ? kt * GBT + r : T - 1;
                const char *sb = (const char *)X + row * K * 2;
                const unsigned off = (c_in && t0 + r < T) ? voff : 0u;
                g[p][r] = *(const u32x4 *)(sb + off);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + r;
                unsigned w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t c0 = cbase + 2 * e;
                    const bool ok0 = t < T && c0 < K, ok1 = t < T && c0 + 1 < K;
                    const unsigned lo = X[ok0 ? t * K + c0 : 0];
                    const unsigned hi = X[ok1 ? t * K + c0 + 1 : 0];
                    w[e] = (ok0 ? lo : 0u) | ((ok1 ? hi : 0u) << 16);
                }
                g[p][r] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    };
    // channel rho = 8 o + c gets tokens 4 q .. 4 q + 3 as one 8-byte word, at
    // byte 8 (q % 2) of chunk q / 2 of its row: physical row 32 c + o, chunk
    // position (q / 2) ^ (c % 4) ^ (o / 8 % 4), i.e. byte 2048 c + sbase[c % 4]
    int sbase[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        sbase[x] = panel * kPanelBytes + 64 * o + 16 * ((q >> 1) ^ x ^ ((o >> 3) & 3)) + 8 * (q & 1);
    auto lstore = [&](auto P, auto SLOT, int64_t kt) {
        constexpr int p = decltype(P)::value;
        int8_t *base = g_lds + 2 * decltype(SLOT)::value * kPanelBytes;
        if constexpr (VEC) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (!(c_in && kt * GBT + 4 * q + r < T)) g[p][r] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // dword e of each token row holds channels 2e (low half) and 2e+1 (high half)
            const unsigned a0 = g[p][0][e], a1 = g[p][1][e], a2 = g[p][2][e], a3 = g[p][3][e];
            const uint2 w0 = make_uint2((a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16));
            const uint2 w1 = make_uint2((a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 2 * e + h;
                *(uint2 *)(base + 2048 * c + sbase[c & 3]) = h ? w1 : w0;
            }
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.0f;

    // operand read offsets (bytes within a panel) for the two k16 halves of a
    // stage: channel rho = r0 + 32 bb + m (r0 a multiple of 32) sits in physical
    // row 32 (m % 8) + r0 / 8 + 4 bb + m / 8, chunk ch at position
    // ch ^ (m % 4) ^ (rho / 64 % 4).  A wave's A rows share rho / 64 = wr; its B
    // rows have rho / 64 = 2 wc + bb / 2.
    const int m = lane & 31;
    int offa[2], offb[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = 2 * h + (lane >> 5);
        const int row = 64 * (32 * (m & 7) + (m >> 3));
        offa[h] = row + 16 * (ch ^ (m & 3) ^ wr) + 512 * wr;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            offb[h][hb] = row + 16 * (ch ^ (m & 3) ^ ((2 * wc + hb) & 3)) + 1024 * wc + 512 * hb;
    }

    // Stage kt: the barrier publishes stage kt (stored during stage kt - 1) and
    // frees the other LDS slot (read during stage kt - 1).  Register set
    // (kt + 1) % 3 holds stage kt + 1 (loaded during stage kt - 3): it goes to
    // LDS, then receives stage kt + 4, so global loads have three stages to
    // land.  The operands of the two k16 halves are read one half at a time
    // (the second while the first half's matrix instructions run).  P (LDS
    // parity), S (register set) and the flags are compile-time, so that the
    // loop body has no branches and the compiler's wait counts stay exact.
    auto step = [&](auto P, auto S, auto STORE, auto LOAD, int64_t kt) {
        constexpr int p = decltype(P)::value, sset = decltype(S)::value;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int8_t *Aq = g_lds + (2 * p) * kPanelBytes, *Bq = g_lds + (2 * p + 1) * kPanelBytes;
        bf16x8 a[2], b[4];
        auto rd = [&](int h) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) a[bb] = *(const bf16x8 *)(Aq + offa[h] + 256 * bb);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) b[bb] = *(const bf16x8 *)(Bq + offb[h][bb >> 1] + 256 * (bb & 1));
        };
        auto mm = [&]() {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
        };
        rd(0);
        if constexpr (decltype(STORE)::value)
            lstore(std::integral_constant<int, sset>{}, std::integral_constant<int, 1 - p>{}, kt + 1);
        if constexpr (decltype(LOAD)::value) gload(std::integral_constant<int, sset>{}, kt + 4);
        __builtin_amdgcn_sched_barrier(0);
        mm();
        __builtin_amdgcn_sched_barrier(0);
        rd(1);
        __builtin_amdgcn_sched_barrier(0);
        mm();
        __builtin_amdgcn_sched_barrier(0);
    };
    using Y = std::true_type;
    using N = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    gload(I0{}, 0);
    gload(I1{}, 1);
    gload(I2{}, 2);
    lstore(I0{}, I0{}, 0);
    gload(I0{}, 3);
    // stage kt uses LDS parity kt % 2 and register set (kt + 1) % 3: a period of 6
    for (int64_t kt = 0; kt < nk - 6; kt += 6) {
        step(I0{}, I1{}, Y{}, Y{}, kt);
        step(I1{}, I2{}, Y{}, Y{}, kt + 1);
        step(I0{}, I0{}, Y{}, Y{}, kt + 2);
        step(I1{}, I1{}, Y{}, Y{}, kt + 3);
        step(I0{}, I2{}, Y{}, Y{}, kt + 4);
        step(I1{}, I0{}, Y{}, Y{}, kt + 5);
    }
    step(I0{}, I1{}, Y{}, Y{}, nk - 6);
    step(I1{}, I2{}, Y{}, Y{}, nk - 5);
    step(I0{}, I0{}, Y{}, N{}, nk - 4);
    step(I1{}, I1{}, Y{}, N{}, nk - 3);
    step(I0{}, I2{}, Y{}, N{}, nk - 2);
    step(I1{}, I0{}, N{}, N{}, nk - 1);

    // H += acc on the lower triangle, one 32 x 32 block at a time (its values
    // of H loaded before any is updated)
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            float h[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = i0 + wr * 64 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int64_t gj = j0 + wc * 128 + bj * 32 + m;
                h[e] = H[(gi < K && gj < K) ? gi * K + gj : 0];
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = i0 + wr * 64 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int64_t gj = j0 + wc * 128 + bj * 32 + m;
                if (gi < K && gj < K && gi >= gj) H[gi * K + gj] = h[e] + acc[bi][bj][e];
            }
        }
}


// ---------------------------------------------------------------------------
// The same product with the activations copied straight from memory into LDS
// (global_load_lds, no registers) and read through the transposing LDS reads of
// gfx950, for K % 8 == 0 and 16-byte aligned chunks.
//
// Four waves of 128 x 128 (2 x 2) on a 256 x 256 lower tile, one wave per
// SIMD, 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 with the sums in AGPRs.  A
// stage is 32 tokens.  In LDS, token row t of a stage holds A's 256 channels
// (512 bytes), then B's (512 bytes), then 64 bytes of padding: one 1 KiB copy
// instruction fills a row (lanes 0..31 A, 32..63 B), and the padding moves each
// row's segments to the next bank group, so the 8 token rows a transposing read
// touches (rows e and 8 + e, e = 0..3, 64 bytes each) take the two passes 512
// bytes need.  ds_read_b64_tr_b16 makes each 16-lane group read a 4 x 16 block
// of 16-bit values (lane 4 e + b: row e, values 4 b .. 4 b + 3) and hands lane
// j column j, i.e. 4 consecutive tokens of one channel; two such reads give the
// 8 tokens of channel l % 32 that lane l feeds the matrix instruction.
//
// Pipeline as in the int8 residue product: a ring of 4 LDS slots, copies three
// stages ahead, one barrier per stage between its two k16 halves, every LDS
// read and copy issued right after one matrix instruction.  Channels past K
// are read from a valid column (their products land only in rows and columns
// of the tile that are never written back); token rows past T are copied from
// a valid row and then overwritten with zeros by the wave that copied them,
// before the barrier that publishes the stage.
//
// Several chunks accumulate in one launch (their pointers and token counts are
// kernel arguments); with more than one split per tile, each split sums its own
// range of chunks and leaves the tile in a partial buffer, which a second
// kernel adds to H in split order, so the result does not depend on timing.
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int RNT = 256, RSLOTS = 4;
constexpr int kRRow = 1088;                         // A 512 | B 512 | pad 64
constexpr int kRSlot = GBT * kRRow;                 // one stage
constexpr size_t kGramRLds = (size_t)RSLOTS * kRSlot;

__device__ inline s16x4 lds_read_tr16(const int8_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
}

// 64 lanes x 16 bytes from g (per lane) to LDS at l + 16 lane, as inline asm so
// that the compiler leaves the waits to wait_vm; M0 is set right before each
// copy and used by nothing else in the kernel.
__device__ inline void gcopy16_lds(const void *g, unsigned l)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l) : "memory");
}
template <int N> __device__ inline void gwait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool DIRECT>
__global__ __launch_bounds__(RNT, 1) void gram_bf16_dma_kernel(float *__restrict__ H, GramChunks ch, int64_t K,
                                                               int splits, float *__restrict__ part)
{
    extern __shared__ __attribute__((aligned(1024))) int8_t r_lds[];
    constexpr int S = RSLOTS;
    const int64_t nt = (K + GBM - 1) / GBM;
    const int64_t ntiles = nt * (nt + 1) / 2;
    const int64_t L = xcd_order(blockIdx.x, gridDim.x);
    const int64_t tile = L % ntiles, split = L / ntiles;
    int64_t ti, tj;
    lower_tile_grouped(tile, nt, ti, tj);
    const int64_t i0 = ti * GBM, j0 = tj * GBM;
    const int c_begin = (int)(split * ch.n / splits), c_end = (int)((split + 1) * ch.n / splits);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    // copies: this wave fills token rows 8 wave + u (u = 0..7) of each stage; lane
    // lane < 32 copies A's chunk lane, the others B's chunk lane - 32
    const int64_t colr = lane < 32 ? i0 + 8 * lane : j0 + 8 * (lane - 32);
    const int64_t col = colr < K ? colr : 0;
    const unsigned lbase = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void *)r_lds +
                           (unsigned)(8 * wave * kRRow);
    // transposing reads: lane l of group g = (l / 16) % 4 reads token row
    // 8 (g / 2) + e (+ 4 for the second read, + 16 for the second k half) and
    // channels 16 (g % 2) + 4 b .. + 3 of a 32-channel block, e = (l % 16) / 4,
    // b = l % 4.  A's blocks start at channel 128 wr + 32 bi, B's at
    // 128 wc + 32 bj.
    const int g4 = (lane >> 4) & 3, e4 = (lane >> 2) & 3, b4 = lane & 3;
    const int lb = kRRow * (8 * (g4 >> 1) + e4) + 32 * (g4 & 1) + 8 * b4;
    const int oa = lb + 256 * wr, ob = lb + 512 + 256 * wc;

    f32x16 acc[4][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[bi][bj][x] = 0.0f;

    for (int c = c_begin; c < c_end; ++c) {
        const uint16_t *__restrict__ X = ch.x[c];
        const int64_t T = ch.t[c];
        if (T <= 0) continue;
        int64_t nk = (T + GBT - 1) / GBT;
        if (nk < S) nk = S;
        const uint16_t *xl = X + col;
        // copy u (token row 8 wave + u) of stage kt into a slot; a row past T
        // copies row T - 1 (it is zeroed before the stage is published)
        auto copy = [&](int64_t kt, int slot, int u) {
            const int64_t t = kt * GBT + 8 * wave + u;
            gcopy16_lds(xl + (t < T ? t : T - 1) * K, lbase + slot * kRSlot + u * kRRow);
        };
        // rows of stage kt that this wave copied past T, to zeros (after its own
        // copies of that stage have landed)
        auto zero_tail = [&](int64_t kt, int slot) {
            if (kt * GBT + 8 * wave + 7 >= T) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                for (int u = 0; u < 8; ++u)
                    if (kt * GBT + 8 * wave + u >= T)
                        *(u32x4 *)(r_lds + slot * kRSlot + (8 * wave + u) * kRRow + 16 * lane) = z;
            }
        };
        auto read = [&](bf16x8 (&a)[4], bf16x8 (&b)[4], int slot, int h, int u) {
            const int8_t *q = r_lds + slot * kRSlot + kRRow * 16 * h;
            const int8_t *p = u < 4 ? q + oa + 64 * u : q + ob + 64 * (u - 4);
            const s16x4 lo = lds_read_tr16(p);
            const s16x4 hi = lds_read_tr16(p + 4 * kRRow);
            const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            if (u < 4) a[u] = v;
            else b[u - 4] = v;
        };
        auto mma = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[4], auto &&side) {
            static_for<16>([&](auto I) {
                constexpr int i = decltype(I)::value;
                acc[i / 4][i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i / 4], b[i % 4], acc[i / 4][i % 4],
                                                                            0, 0, 0);
                side(I);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        bf16x8 a0[4], b0[4], a1[4], b1[4];
        // Stage kt, entered with stage kt published and its first-half operands in
        // a0/b0 (or on their way): first half, reading the second half's operands
        // and copying rows 0..3 of stage kt + S - 1 into the slot of stage kt - 1
        // (free: its last reads, in stage kt - 1's first half and stage kt - 2's
        // second, came before stage kt - 1's barrier); wait for this wave's copies
        // of stage kt + 1, zero its rows past T, barrier (stage kt + 1
        // published); second half, reading stage kt + 1's first-half operands
        // and copying rows 4..7 of stage kt + S - 1.
        auto step = [&](auto WN, auto C, auto NEXT, int64_t kt, int slot) {
            const int nslot = slot == S - 1 ? 0 : slot + 1;
            const int fslot = slot == 0 ? S - 1 : slot - 1;        // slot of stages kt - 1 and kt + S - 1
            mma(a0, b0, [&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i % 2 == 0) read(a1, b1, slot, 1, i / 2);
                else if constexpr (decltype(C)::value && i % 4 == 1) copy(kt + S - 1, fslot, i / 4);
            });
            if constexpr (decltype(NEXT)::value) {
                gwait_vm<decltype(WN)::value>();
                zero_tail(kt + 1, nslot);
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            __builtin_amdgcn_sched_barrier(0);
            mma(a1, b1, [&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (decltype(NEXT)::value) {
                    if constexpr (i % 2 == 0) read(a0, b0, nslot, 0, i / 2);
                    else if constexpr (decltype(C)::value && i % 4 == 1) copy(kt + S - 1, fslot, 4 + i / 4);
                }
            });
        };
        using Tt = std::true_type;
        using Ff = std::false_type;
        // the previous chunk's last stages may still be read from the slots
        __syncthreads();
        // prologue: stages 0 .. S - 2 whole
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
#pragma unroll
            for (int u = 0; u < 8; ++u) copy(st, st, u);
        gwait_vm<8 * (S - 2)>();
        zero_tail(0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int u = 0; u < 8; ++u) read(a0, b0, 0, 0, u);
        int slot = 0;
        int64_t kt = 0;
        // Stage j is copied during stage j - S + 1 (rows 0..3 in its first half,
        // 4..7 in its second), so at stage kt's barrier, which needs stage kt + 1,
        // this wave's newer copies are those of stages kt + 2 .. kt + S - 2 and
        // the first four of stage kt + S - 1: 8 (S - 3) + 4 may stay in flight.
        // Near the end no copies are issued and the count falls by 8 per stage.
        for (; kt <= nk - S; ++kt) {
            step(std::integral_constant<int, 8 * (S - 3) + 4>{}, Tt{}, Tt{}, kt, slot);
            slot = slot == S - 1 ? 0 : slot + 1;
        }
        static_for<S - 2>([&](auto J) {
            constexpr int j = decltype(J)::value;
            step(std::integral_constant<int, 8 * (S - 3 - j)>{}, Ff{}, Tt{}, kt, slot);
            ++kt;
            slot = slot == S - 1 ? 0 : slot + 1;
        });
        step(std::integral_constant<int, 0>{}, Ff{}, Ff{}, kt, slot);
    }

    const int m = lane & 31;
    if constexpr (DIRECT) {
        // H += acc on the lower triangle, one 32 x 32 block at a time: its 16
        // values of H are loaded (from clamped addresses) before any is
        // updated, so the tile waits on memory once per block, not per element
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                float h[16];
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int64_t gi = i0 + wr * 128 + bi * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
                    const int64_t gj = j0 + wc * 128 + bj * 32 + m;
                    h[x] = H[(gi < K && gj < K) ? gi * K + gj : 0];
                }
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int64_t gi = i0 + wr * 128 + bi * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
                    const int64_t gj = j0 + wc * 128 + bj * 32 + m;
                    if (gi < K && gj < K && gi >= gj) H[gi * K + gj] = h[x] + acc[bi][bj][x];
                }
            }
    } else {
        // this split's tile, thread-major: 256 floats per thread
        float4 *dst = (float4 *)(part + ((tile * splits + split) * RNT + tid) * 256);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                for (int x = 0; x < 16; x += 4)
                    dst[(bi * 4 + bj) * 4 + x / 4] =
                        make_float4(acc[bi][bj][x], acc[bi][bj][x + 1], acc[bi][bj][x + 2], acc[bi][bj][x + 3]);
    }
}

// H += the splits' partial tiles, summed in split order.  One workgroup per
// tile, thread tid of the product kernel's layout.
__global__ __launch_bounds__(RNT) void gram_split_sum_kernel(float *__restrict__ H, const float *__restrict__ part,
                                                             int64_t K, int splits)
{
    const int64_t nt = (K + GBM - 1) / GBM;
    const int64_t tile = blockIdx.x;
    int64_t ti, tj;
    lower_tile_grouped(tile, nt, ti, tj);
    const int64_t i0 = ti * GBM, j0 = tj * GBM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1, m = lane & 31;
    for (int blk = 0; blk < 16; ++blk) {
        const int bi = blk >> 2, bj = blk & 3;
        float sum[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) sum[x] = 0.0f;
        for (int s = 0; s < splits; ++s) {
            const float4 *src = (const float4 *)(part + ((tile * splits + s) * RNT + tid) * 256) + blk * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 q = src[v];
                sum[4 * v] += q.x;
                sum[4 * v + 1] += q.y;
                sum[4 * v + 2] += q.z;
                sum[4 * v + 3] += q.w;
            }
        }
        float h[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int64_t gi = i0 + wr * 128 + bi * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
            const int64_t gj = j0 + wc * 128 + bj * 32 + m;
            h[x] = H[(gi < K && gj < K) ? gi * K + gj : 0];
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int64_t gi = i0 + wr * 128 + bi * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
            const int64_t gj = j0 + wc * 128 + bj * 32 + m;
            if (gi < K && gj < K && gi >= gj) H[gi * K + gj] = h[x] + sum[x];
        }
    }
}

}  // namespace

hipError_t launch_gram_bf16(float *H, const uint16_t *X, int64_t T, int64_t K, hipStream_t s)
{
    if (T <= 0 || K <= 0) return hipSuccess;
    if ((K % 8 == 0) && (((uintptr_t)X & 15) == 0)) {
        GramChunks ch{};
        ch.x[0] = X;
        ch.t[0] = T;
        ch.n = 1;
        return launch_gram_bf16_chunks(H, ch, K, 1, nullptr, s);
    }
    static const bool lds_ok =
        hipFuncSetAttribute((const void *)gram_bf16_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kGramLds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int64_t nt = (K + GBM - 1) / GBM;
    const dim3 grid((unsigned)(nt * (nt + 1) / 2));
    hipLaunchKernelGGL(gram_bf16_kernel<false>, grid, dim3(GNT), kGramLds, s, H, X, T, K);
    return hipGetLastError();
}

int64_t gram_tiles(int64_t K)
{
    const int64_t nt = (K + GBM - 1) / GBM;
    return nt * (nt + 1) / 2;
}

size_t gram_split_bytes(int64_t K, int splits)
{
    return splits > 1 ? (size_t)gram_tiles(K) * (size_t)splits * GBM * GBM * sizeof(float) : 0;
}

hipError_t launch_gram_bf16_chunks(float *H, const GramChunks &ch, int64_t K, int splits, float *part, hipStream_t s)
{
    if (K <= 0 || ch.n <= 0) return hipSuccess;
    if (splits < 1 || splits > ch.n || (splits > 1 && !part)) return hipErrorInvalidValue;
    static const bool lds_ok =
        hipFuncSetAttribute((const void *)gram_bf16_dma_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kGramRLds) == hipSuccess &&
        hipFuncSetAttribute((const void *)gram_bf16_dma_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kGramRLds) == hipSuccess;
    if (!lds_ok) return hipErrorInvalidConfiguration;
    const int64_t tiles = gram_tiles(K);
    const dim3 grid((unsigned)(tiles * splits));
    if (splits == 1) {
        hipLaunchKernelGGL(gram_bf16_dma_kernel<true>, grid, dim3(RNT), kGramRLds, s, H, ch, K, 1, nullptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(gram_bf16_dma_kernel<false>, grid, dim3(RNT), kGramRLds, s, H, ch, K, splits, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gram_split_sum_kernel, dim3((unsigned)tiles), dim3(RNT), 0, s, H, part, K, splits);
    return hipGetLastError();
}

}  // namespace gq
