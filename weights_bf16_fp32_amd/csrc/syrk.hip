// Covariance aggregation C <- beta C + alpha X^T X (lower triangle), gfx950.
//
// The second-moment matrix S = (1/n) X^T X of the Marchenko-Pastur setting and
// the window covariance of EigenTrack ("Random matrix theory spectral methods"
// page, sections 2.1 and 3.1), summed block by block as Swift-SVD's incremental
// covariance aggregation (Swift-SVD page, sections 2 and 7).
//
// Kernels
//   syrk_bf16_mfma  bf16 X, fp32 C.  128x128 lower-triangle tiles of C, one
//                   workgroup (4 waves, 64x64 each) per tile, K-loop over the
//                   samples in steps of 64.  X is row-major with the reduction
//                   index (samples) as the slow dimension, while the MFMA wants
//                   8 consecutive samples per lane, so each thread loads an 8x8
//                   (samples x features) block with 16-byte loads, transposes it
//                   in registers and stores feature-major rows into LDS.  LDS is
//                   double-buffered; the next block's global loads are in flight
//                   during the current block's MFMAs.  v_mfma_f32_32x32x16_bf16.
//   syrk_f64_mfma   f32 X, fp64 C.  Products of two f32 values are exact in
//                   fp64; v_mfma_f64_16x16x4_f64 accumulates them.  The MFMA
//                   takes one sample per lane, so X's natural layout is used
//                   as is (converted to fp64 on the way into LDS).
//   syrk_generic    any of the above pairs plus f32 -> f32, plain VALU FMAs on
//                   64x64 tiles; used for f32 -> f32 and for shapes the MFMA
//                   kernels do not take (d or ldx not a multiple of 8).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int SB_TILE = 128;  // C tile edge
constexpr int SB_BK = 64;     // samples per K-step
constexpr int SB_LDS_ROW = 72;  // uint16 per LDS row: 64 samples + 8 pad (144 B)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__global__ __launch_bounds__(256) void syrk_bf16_mfma(const uint16_t *__restrict__ X, int64_t n, int64_t d,
                                                      int64_t ldx, float *__restrict__ C, int64_t ldc, float alpha,
                                                      float beta)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][SB_TILE * SB_LDS_ROW];

    int ti, tj;
    tri_tile_blocked(xcd_remap(blockIdx.x, gridDim.x), (int)((d + SB_TILE - 1) / SB_TILE), ti, tj);
    const int64_t i0 = (int64_t)ti * SB_TILE, j0 = (int64_t)tj * SB_TILE;
    const bool diag = ti == tj;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // loader role: operand (0 = rows of C, 1 = columns of C), 8-feature block, 8-sample block
    const int op = tid >> 7;
    const int fb = (tid & 127) >> 3;
    const int kb = tid & 7;
    const bool loader = !(diag && op == 1);
    const int64_t fbase = (op == 0 ? i0 : j0) + fb * 8;
    const bool f_ok = fbase < d;  // d % 8 == 0: a block is wholly inside or outside

    // v[e] holds samples (k0 + 8 kb + e), features fbase .. fbase + 7 (two per word).
    // Buffer loads from a resource that starts at sample k0 and ends at sample
    // n: rows past the end read as zero, and a feature block past d gets an
    // offset beyond every resource, so no load is predicated.
    const uint32_t ldb = (uint32_t)(ldx * 2);  // bytes per sample
    uint32_t voff[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        voff[e] = f_ok && loader ? (uint32_t)(kb * 8 + e) * ldb + (uint32_t)fbase * 2u : 0xFFFFFFF0u;
    // four register stages: the samples of step k + 3 are requested while step k
    // runs on MFMA, and written to LDS two steps later, so a load has three
    // steps to arrive
    constexpr int PF = 4;
    u32x4_t vb[PF][8];
    auto gload = [&](u32x4_t (&v)[8], int64_t k0) {
        const int64_t rem = (n - k0) * ldx * 2;  // bytes from sample k0 to the end (<= 0: none)
        const int num = (int)(rem <= 0 ? 0 : (rem < 0x7FFFFFF0 ? rem : 0x7FFFFFF0));
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(X + (rem > 0 ? k0 : 0) * ldx), 0, num, 0x00020000);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[e], 0, 0));
    };
    // transpose: LDS row (feature f) gets samples 8 kb .. 8 kb + 7 (two per word),
    // each word one byte permute of two loaded words
    auto lstore = [&](const u32x4_t (&v)[8], int stage) {
        uint16_t *base = &lds[stage][op][0] + (fb * 8) * SB_LDS_ROW + kb * 8;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                o[p] = __builtin_amdgcn_perm(v[2 * p + 1][f >> 1], v[2 * p][f >> 1],
                                             (f & 1) ? 0x07060302u : 0x05040100u);
            *reinterpret_cast<u32x4_t *>(base + f * SB_LDS_ROW) = o;
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    const bool active = !(diag && wm == 0 && wn == 1);  // strictly upper quadrant of a diagonal tile
    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    // Every thread loads and stores unconditionally (straight-line code lets the
    // compiler wait for exactly the stage it needs): the second operand's
    // threads of a diagonal tile read zeros and write them to the operand half
    // that tile never reads.
#pragma unroll
    for (int p = 0; p < PF - 1; ++p) gload(vb[p], p * SB_BK);
    lstore(vb[0], 0);
    __syncthreads();
    // fragment rows of this lane in both operands (a diagonal tile reads its one operand twice)
    const uint16_t *fa_base = &lds[0][0][0] + (wm * 64 + (lane & 31)) * SB_LDS_ROW + (lane >> 5) * 8;
    const uint16_t *fb_base = &lds[0][diag ? 0 : 1][0] + (wn * 64 + (lane & 31)) * SB_LDS_ROW + (lane >> 5) * 8;
    constexpr int STAGE = 2 * SB_TILE * SB_LDS_ROW;  // uint16 per stage
    // steps past n read zeros and add nothing, so the step count is rounded up to PF
    const int64_t nsteps = (n + SB_BK - 1) / SB_BK;
    for (int64_t s0 = 0; s0 < nsteps; s0 += PF) {
        static_for<0, PF>([&](auto UC) {
            constexpr int u = decltype(UC)::value;
            const int64_t k = s0 + u;
            gload(vb[(u + PF - 1) % PF], (k + PF - 1) * SB_BK);
            // every wave runs its MFMAs (the upper quadrant of a diagonal tile is
            // computed and not stored), so the accumulators need no copies
            const uint16_t *la = fa_base + (u & 1) * STAGE, *lb = fb_base + (u & 1) * STAGE;
#pragma unroll
            for (int kk = 0; kk < SB_BK / 16; ++kk) {
                bf16x8_t fa[2], fbv[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    fa[m] = *reinterpret_cast<const bf16x8_t *>(la + m * 32 * SB_LDS_ROW + kk * 16);
                    fbv[m] = *reinterpret_cast<const bf16x8_t *>(lb + m * 32 * SB_LDS_ROW + kk * 16);
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fbv[b], acc[a][b], 0, 0, 0);
            }
            lstore(vb[(u + 1) % PF], (u + 1) & 1);
            __syncthreads();
        });
    }

    if (!active) return;
    // every old value of C is loaded before the first store, so the loads are in
    // flight together instead of one read-modify-write round trip at a time
    auto rc = [&](int a, int b, int e, int64_t &row, int64_t &col) {
        col = j0 + wn * 64 + b * 32 + (lane & 31);
        row = i0 + wm * 64 + a * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        return row < d && col < d && row >= col;
    };
    if (beta != 0.f) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    int64_t row, col;
                    const float old = rc(a, b, e, row, col) ? C[row * ldc + col] : 0.f;
                    acc[a][b][e] = alpha * acc[a][b][e] + beta * old;
                }
    } else {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] *= alpha;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int64_t row, col;
                if (rc(a, b, e, row, col)) C[row * ldc + col] = acc[a][b][e];
            }
}

// ---------------------------------------------------------------- bf16 MFMA, 256 x 256 tiles
//
// syrk_bf16_big: the same product for large d.  A 128 x 128 tile reads two
// 128-feature strips of X per 128^2 outputs, and at d = 14336 the concurrent
// tiles of an XCD hit its L2 only a quarter of the time, so the kernel streamed
// X from HBM ~77 times.  Here a tile is 256 x 256 (4 waves of 128 x 128, 16
// accumulator blocks of 32 x 32 each, all in AGPRs), which halves the strip
// reads per output.  One workgroup per CU runs at a time (all 512 registers
// of a lane), so the tiles run in rounds of one workgroup per CU, started
// together and of equal cost; in round r, workgroup b (dealt to XCD b % 8)
// takes tile r * R + (b % 8) * (R / 8) + (b mod R) / 8 of the blocked
// triangle order (R = CUs per round), so the 32 tiles an XCD runs together
// form a 4 x 8 block of one 8 x 8 super-block (12 strips) and advance through
// the samples in step.
// LDS: per operand and stage, sample group g (8 samples, 16 bytes per feature)
// holds 256 features, feature f in 16-byte slot f ^ ((f >> 3) & 15): the
// operand reads (16 consecutive features) and the loader's writes (features
// 8 apart, f = 8 fb + c) both land on 16 distinct slots modulo 16, so neither
// conflicts whether the hardware serves 8 lanes on 32 banks or 16 lanes on 64.
constexpr int BG_TILE = 256;
constexpr int BG_BK = 32;                               // samples per K-step
constexpr int BG_GROUP_U16 = BG_TILE * 8;               // uint16 per sample group (4 KB)
constexpr int BG_OP_U16 = (BG_BK / 8) * BG_GROUP_U16;   // one operand, one stage
constexpr int BG_PF = 3;                                // register stages of prefetch

__device__ __forceinline__ int bg_slot(int f) { return (f ^ ((f >> 3) & 15)) * 8; }  // uint16 offset of feature f

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void syrk_bf16_big(const uint16_t *__restrict__ X, int64_t n, int64_t d,
                                                     int64_t ldx, float *__restrict__ C, int64_t ldc, float alpha,
                                                     float beta, int64_t ntiles, int round, int64_t tile0, int splits)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BG_OP_U16];
    const int nt = (int)((d + BG_TILE - 1) / BG_TILE);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // loader: operand op, 8-feature block fb (0..31), 8-sample group kb (0..3)
    const int fb = tid & 31, kb = (tid >> 5) & 3, op = tid >> 7;
    const uint32_t ldb = (uint32_t)(ldx * 2);
    // splits == 1: tiles 0 .. ntiles-1 in rounds (below); splits > 1: workgroup
    // b takes tile tile0 + b / splits over its share of the K-steps and adds
    // alpha times its partial product to C atomically (C was scaled by beta)
    const int64_t nsteps_all = (n + BG_BK - 1) / BG_BK;
    const int sp = splits > 1 ? (int)(blockIdx.x % splits) : 0;
    const int64_t per = (nsteps_all + splits - 1) / splits;
    const int64_t n_begin = min<int64_t>(n, sp * per * BG_BK);
    const int64_t n_end = min<int64_t>(n, (sp + 1) * per * BG_BK);
    const int64_t nsteps = (n_end - n_begin + BG_BK - 1) / BG_BK;
    // rounds of `round` consecutive workgroups run together (one per CU); in a
    // full round, the hardware deals workgroup b to XCD b % 8, and that XCD's
    // round/8 workgroups take consecutive tiles of the blocked order
    const int64_t b = blockIdx.x;
    const int64_t r0 = b / round * round;
    const int64_t t = splits > 1 ? tile0 + b / splits
                                 : (r0 + round <= ntiles ? r0 + (b % 8) * (round / 8) + (b - r0) / 8 : b);
    {
        int ti, tj;
        tri_tile_blocked(t, nt, ti, tj);
        const int64_t i0 = (int64_t)ti * BG_TILE, j0 = (int64_t)tj * BG_TILE;
        const bool diag = ti == tj;
        const bool loader = !(diag && op == 1);
        const int64_t fbase = (op == 0 ? i0 : j0) + fb * 8;
        uint32_t voff[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            voff[e] = fbase < d && loader ? (uint32_t)(kb * 8 + e) * ldb + (uint32_t)fbase * 2u : 0xFFFFFFF0u;
        u32x4_t vb[BG_PF][8];
        auto gload = [&](u32x4_t (&v)[8], int64_t kr) {
            const int64_t k0 = n_begin + kr;  // first sample of the K-step
            const int64_t rem = (n_end - k0) * ldx * 2;
            const int num = (int)(rem <= 0 ? 0 : (rem < 0x7FFFFFF0 ? rem : 0x7FFFFFF0));
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void *)(X + (rem > 0 ? k0 : 0) * ldx), 0, num, 0x00020000);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[e], 0, 0));
        };
        auto lstore = [&](const u32x4_t (&v)[8], int stage) {
            uint16_t *base = &lds[stage][op][0] + kb * BG_GROUP_U16;
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                u32x4_t o;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    o[p] = __builtin_amdgcn_perm(v[2 * p + 1][f >> 1], v[2 * p][f >> 1],
                                                 (f & 1) ? 0x07060302u : 0x05040100u);
                *reinterpret_cast<u32x4_t *>(base + bg_slot(fb * 8 + f)) = o;
            }
        };
        f32x16_t acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
        const bool active = !(diag && wm == 0 && wn == 1);
#pragma unroll
        for (int p = 0; p < BG_PF - 1; ++p) gload(vb[p], p * BG_BK);
        lstore(vb[0], 0);
        __syncthreads();
        // operand rows of this lane: A rows wm*128 + a*32 + l%32, B rows wn*128 + b*32 + l%32;
        // sample group 2 kk + l / 32 of the K-step
        const int gsel = (lane >> 5) * BG_GROUP_U16;
        for (int64_t s0 = 0; s0 < nsteps; s0 += BG_PF) {
            static_for<0, BG_PF>([&](auto UC) {
                constexpr int u = decltype(UC)::value;
                const int64_t k = s0 + u;
                gload(vb[(u + BG_PF - 1) % BG_PF], (k + BG_PF - 1) * BG_BK);
                const int st = (int)(k & 1);
                const uint16_t *la = &lds[st][0][0] + gsel;
                const uint16_t *lb = &lds[st][diag ? 0 : 1][0] + gsel;
                // every wave computes (on a diagonal tile the block above the
                // diagonal is computed and dropped at the store), so the step is
                // one basic block: the loads, the first K-half's operands, its 16
                // MFMAs each with two permutes of the next stage, the second
                // K-half's operands, its 16 MFMAs with the LDS writes
#pragma unroll
                for (int kk = 0; kk < BG_BK / 16; ++kk) {
                    bf16x8_t fa[4], fbv[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        fa[m] = *reinterpret_cast<const bf16x8_t *>(
                            la + 2 * kk * BG_GROUP_U16 + bg_slot(wm * 128 + m * 32 + (lane & 31)));
                        fbv[m] = *reinterpret_cast<const bf16x8_t *>(
                            lb + 2 * kk * BG_GROUP_U16 + bg_slot(wn * 128 + m * 32 + (lane & 31)));
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fbv[b], acc[a][b], 0, 0, 0);
                }
                lstore(vb[(u + 1) % BG_PF], st ^ 1);
                __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                static_for<0, 16>([&](auto) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                });
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                static_for<0, 8>([&](auto) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                });
                static_for<0, 8>([&](auto) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); });
                __syncthreads();
            });
        }
        if (active) {
            // C through a buffer resource from the tile's corner to the end of the
            // matrix: 32-bit offsets (ldc < 2^21 is checked by the launcher), one
            // VGPR per element; an element outside the lower triangle or past d
            // gets an offset beyond every resource (its load reads 0, its store
            // is dropped).  Four accumulator blocks at a time, their old values
            // all loaded before the first store.
            const int64_t corner = i0 * ldc + j0;
            const int64_t span = ((d - 1) * ldc + d - corner) * 4;
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc(C + corner, 0, (int)(span < 0x7FFFFFF0 ? span : 0x7FFFFFF0),
                                                  0x00020000);
            const int ldc4 = (int)ldc * 4;
            const int rl = wm * 128 + (lane >> 5) * 4, cl = wn * 128 + (lane & 31);
            const uint32_t lane_off = (uint32_t)(rl * ldc4 + cl * 4);
            const int rlim = (int)min<int64_t>(d - i0, BG_TILE), clim = (int)min<int64_t>(d - j0, BG_TILE);
            // one 32 x 32 block at a time: its 16 old values (beta != 0) are loaded
            // before its 16 stores
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    uint32_t off[16];
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int dr = a * 32 + (e >> 2) * 8 + (e & 3);
                        const int row = rl + dr, col = cl + b * 32;  // within the tile
                        const bool ok = row < rlim && col < clim && (!diag || row >= col);
                        off[e] = ok ? lane_off + (uint32_t)(dr * ldc4 + b * 128) : 0x80000000u;
                    }
                    float v[16];
                    if (splits > 1) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(alpha * acc[a][b][e], rc, (int)off[e], 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        continue;
                    }
                    if (beta != 0.f) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)off[e], 0, 0));
#pragma unroll
                        for (int e = 0; e < 16; ++e) v[e] = alpha * acc[a][b][e] + beta * v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) v[e] = alpha * acc[a][b][e];
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[e]), rc, (int)off[e], 0, 0);
                    __builtin_amdgcn_sched_barrier(0);  // one block's values live at a time
                }
        }
    }
}

// ---------------------------------------------------------------- fp64 MFMA

constexpr int SD_TILE = 128;
constexpr int SD_BK = 16;
constexpr int SD_LDS_ROW = SD_TILE + 2;  // doubles per LDS row (pad 16 B)

__global__ __launch_bounds__(256) void syrk_f64_mfma(const float *__restrict__ X, int64_t n, int64_t d, int64_t ldx,
                                                     double *__restrict__ C, int64_t ldc, double alpha, double beta)
{
    __shared__ __attribute__((aligned(16))) double lds[2][2][SD_BK * SD_LDS_ROW];

    int ti, tj;
    tri_tile_blocked(xcd_remap(blockIdx.x, gridDim.x), (int)((d + SD_TILE - 1) / SD_TILE), ti, tj);
    const int64_t i0 = (int64_t)ti * SD_TILE, j0 = (int64_t)tj * SD_TILE;
    const bool diag = ti == tj;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // loader: operand op = tid >> 7; each thread loads 2 x float4 (rows kr, kr + 8; 4 features)
    const int op = tid >> 7;
    const int u = tid & 127;
    const int fq = u & 31;       // 4-feature group within the 128 features
    const int kr = u >> 5;       // 0..3 -> rows kr, kr+4, kr+8, kr+12
    const bool loader = !(diag && op == 1);
    const int64_t fbase = (op == 0 ? i0 : j0) + fq * 4;
    const bool f_ok = fbase < d;  // d % 4 == 0

    float4 v[4];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int64_t k = k0 + kr + 4 * e;
            if (loader && f_ok && k < n)
                v[e] = *reinterpret_cast<const float4 *>(X + k * ldx + fbase);
            else
                v[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto lstore = [&](int stage) {
        if (!loader) return;
        double *base = &lds[stage][op][0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double *p = base + (kr + 4 * e) * SD_LDS_ROW + fq * 4;
            p[0] = (double)v[e].x;
            p[1] = (double)v[e].y;
            p[2] = (double)v[e].z;
            p[3] = (double)v[e].w;
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    const bool active = !(diag && wm == 0 && wn == 1);
    f64x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f64x4_t{0.0, 0.0, 0.0, 0.0};

    gload(0);
    lstore(0);
    __syncthreads();
    int cur = 0;
    for (int64_t k0 = 0; k0 < n; k0 += SD_BK) {
        const bool more = k0 + SD_BK < n;
        if (more) gload(k0 + SD_BK);
        if (active) {
            const double *la = &lds[cur][0][0];
            const double *lb = &lds[cur][diag ? 0 : 1][0];
#pragma unroll
            for (int kk = 0; kk < SD_BK / 4; ++kk) {
                const int krow = kk * 4 + (lane >> 4);
                double fa[4], fbv[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) fa[m] = la[krow * SD_LDS_ROW + wm * 64 + m * 16 + (lane & 15)];
#pragma unroll
                for (int m = 0; m < 4; ++m) fbv[m] = lb[krow * SD_LDS_ROW + wn * 64 + m * 16 + (lane & 15)];
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[a], fbv[b], acc[a][b], 0, 0, 0);
            }
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }
    if (!active) return;
    // v_mfma_f64_16x16x4f64 result: lane l holds column l % 16, rows l / 16 + 4 e.
    // All old values are loaded before the first store.
    auto rc = [&](int a, int b, int e, int64_t &row, int64_t &col) {
        col = j0 + wn * 64 + b * 16 + (lane & 15);
        row = i0 + wm * 64 + a * 16 + (lane >> 4) + 4 * e;
        return row < d && col < d && row >= col;
    };
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int64_t row, col;
                const double old = beta != 0.0 && rc(a, b, e, row, col) ? C[row * ldc + col] : 0.0;
                acc[a][b][e] = alpha * acc[a][b][e] + beta * old;
            }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int64_t row, col;
                if (rc(a, b, e, row, col)) C[row * ldc + col] = acc[a][b][e];
            }
}

// ---------------------------------------------------------------- generic VALU

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn *p);
template <>
__device__ __forceinline__ float load_in<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

constexpr int SG_TILE = 64;
constexpr int SG_BK = 16;

template <typename TIn, typename TAcc>
__global__ __launch_bounds__(256) void syrk_generic(const TIn *__restrict__ X, int64_t n, int64_t d, int64_t ldx,
                                                    TAcc *__restrict__ C, int64_t ldc, TAcc alpha, TAcc beta)
{
    __shared__ TAcc As[SG_BK][SG_TILE + 1], Bs[SG_BK][SG_TILE + 1];
    int ti, tj;
    tri_tile(blockIdx.x, ti, tj);
    const int64_t i0 = (int64_t)ti * SG_TILE, j0 = (int64_t)tj * SG_TILE;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    TAcc acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0;
    for (int64_t k0 = 0; k0 < n; k0 += SG_BK) {
        for (int idx = threadIdx.x; idx < SG_BK * SG_TILE; idx += 256) {
            int kk = idx / SG_TILE, f = idx % SG_TILE;
            int64_t k = k0 + kk;
            TAcc va = 0, vb = 0;
            if (k < n && i0 + f < d) va = (TAcc)load_in<TIn>(X + k * ldx + i0 + f);
            if (k < n && j0 + f < d) vb = (TAcc)load_in<TIn>(X + k * ldx + j0 + f);
            As[kk][f] = va;
            Bs[kk][f] = vb;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < SG_BK; ++kk) {
            TAcc a[4], b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = As[kk][ty * 4 + e];
                b[e] = Bs[kk][tx * 4 + e];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] += a[p] * b[q];
        }
        __syncthreads();
    }
    // all old values are loaded before the first store
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = i0 + ty * 4 + p, col = j0 + tx * 4 + q;
            const bool in = row < d && col < d && row >= col;
            const TAcc old = beta != (TAcc)0 && in ? C[row * ldc + col] : (TAcc)0;
            acc[p][q] = alpha * acc[p][q] + beta * old;
        }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = i0 + ty * 4 + p, col = j0 + tx * 4 + q;
            if (row < d && col < d && row >= col) C[row * ldc + col] = acc[p][q];
        }
}

inline int64_t tri_count(int64_t t) { return t * (t + 1) / 2; }

}  // namespace

// C <- beta C on the lower triangle of 256 x 256 tiles tile0 .. tile0 + count - 1
// (blocked order), before their split-K partial products are added
__global__ __launch_bounds__(256) void syrk_scale_tiles(float *__restrict__ C, int64_t ldc, int64_t d, float beta,
                                                        int64_t tile0)
{
    const int nt = (int)((d + BG_TILE - 1) / BG_TILE);
    int ti, tj;
    tri_tile_blocked(tile0 + blockIdx.x, nt, ti, tj);
    const int64_t i0 = (int64_t)ti * BG_TILE, j0 = (int64_t)tj * BG_TILE;
    const int64_t c = j0 + threadIdx.x;
    for (int r = 0; r < BG_TILE; ++r) {
        const int64_t i = i0 + r;
        if (i < d && c < d && c <= i) {
            float *p = C + i * ldc + c;
            *p = beta == 0.f ? 0.f : beta * *p;
        }
    }
}

hipError_t launch_syrk(hipStream_t stream, const void *X, int xt, int64_t n, int64_t d, int64_t ldx, void *C, int ct,
                       int64_t ldc, double alpha, double beta)
{
    if (xt == SPEC_BF16 && ct == SPEC_F32) {
        // the MFMA kernel addresses 64 samples from one buffer base with 32-bit
        // offsets: 64 * ldx * 2 bytes must stay below the resource limit
        const bool vec = d % 8 == 0 && ldx % 8 == 0 && ((uintptr_t)X % 16) == 0 && ldx <= ((int64_t)1 << 24) - 8;
        const int64_t big_tiles = tri_count((d + BG_TILE - 1) / BG_TILE);
        hipDevice_t dev = 0;
        int cus = 256;
        if (hipStreamGetDevice(stream, &dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const int round = cus >= 8 ? cus / 8 * 8 : 8;
        if (vec && big_tiles >= round / 2 && ldc < ((int64_t)1 << 21)) {
            // large d: 256 x 256 tiles in rounds of one workgroup per CU
            int64_t full, tail;
            int splits = 1;
            if (big_tiles >= round) {
                // full rounds as they are; a last round under half full is split along
                // the samples (up to 4 ways, the partial products added atomically)
                // so that its workgroups fill the chip
                full = big_tiles / round * round;
                tail = big_tiles - full;
                splits = tail > 0 && tail <= round / 2 ? (int)std::min<int64_t>(4, round / tail) : 1;
            } else {
                // fewer tiles than CUs (d from 3848 to 5632 on 256 CUs): every tile split
                // the same number of ways (up to 8, at least 4096 samples each),
                // the count whose rounds are fullest
                full = 0;
                tail = big_tiles;
                double best = 0.0;
                for (int s = 1; s <= 8 && (s == 1 || n / s >= 4096); ++s) {
                    const int64_t wgs = big_tiles * s, rounds = (wgs + round - 1) / round;
                    const double fill = (double)wgs / (double)(rounds * round);
                    if (fill > best + 0.02) {
                        best = fill;
                        splits = s;
                    }
                }
            }
            const int64_t main = splits > 1 ? full : big_tiles;
            if (main > 0)
                hipLaunchKernelGGL(syrk_bf16_big, dim3((unsigned)main), dim3(256), 0, stream, (const uint16_t *)X, n,
                                   d, ldx, (float *)C, ldc, (float)alpha, (float)beta, main, round, (int64_t)0, 1);
            if (splits > 1) {
                hipLaunchKernelGGL(syrk_scale_tiles, dim3((unsigned)tail), dim3(256), 0, stream, (float *)C, ldc, d,
                                   (float)beta, full);
                hipLaunchKernelGGL(syrk_bf16_big, dim3((unsigned)(tail * splits)), dim3(256), 0, stream,
                                   (const uint16_t *)X, n, d, ldx, (float *)C, ldc, (float)alpha, (float)beta, tail,
                                   round, full, splits);
            }
        } else if (vec) {
            int64_t tiles = tri_count((d + SB_TILE - 1) / SB_TILE);
            hipLaunchKernelGGL(syrk_bf16_mfma, dim3((unsigned)tiles), dim3(256), 0, stream, (const uint16_t *)X, n, d,
                               ldx, (float *)C, ldc, (float)alpha, (float)beta);
        } else {
            int64_t tiles = tri_count((d + SG_TILE - 1) / SG_TILE);
            hipLaunchKernelGGL((syrk_generic<uint16_t, float>), dim3((unsigned)tiles), dim3(256), 0, stream,
                               (const uint16_t *)X, n, d, ldx, (float *)C, ldc, (float)alpha, (float)beta);
        }
    } else if (xt == SPEC_F32 && ct == SPEC_F32) {
        int64_t tiles = tri_count((d + SG_TILE - 1) / SG_TILE);
        hipLaunchKernelGGL((syrk_generic<float, float>), dim3((unsigned)tiles), dim3(256), 0, stream,
                           (const float *)X, n, d, ldx, (float *)C, ldc, (float)alpha, (float)beta);
    } else if (xt == SPEC_F32 && ct == SPEC_F64) {
        if (d % 4 == 0 && ldx % 4 == 0 && ((uintptr_t)X % 16) == 0) {
            int64_t tiles = tri_count((d + SD_TILE - 1) / SD_TILE);
            hipLaunchKernelGGL(syrk_f64_mfma, dim3((unsigned)tiles), dim3(256), 0, stream, (const float *)X, n, d, ldx,
                               (double *)C, ldc, alpha, beta);
        } else {
            int64_t tiles = tri_count((d + SG_TILE - 1) / SG_TILE);
            hipLaunchKernelGGL((syrk_generic<float, double>), dim3((unsigned)tiles), dim3(256), 0, stream,
                               (const float *)X, n, d, ldx, (double *)C, ldc, alpha, beta);
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
