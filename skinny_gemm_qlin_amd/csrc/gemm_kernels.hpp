// gemm_kernels.hpp -- tiled matrix-core GEMM for prefill-sized M (> 16),
// the same four dense contracts as the decode kernels:
//   INT8 W8A8        y = bf16((acc * xs[m]) * ws[n]) (+ bias), acc exact int32
//                    [Z100 operator-family table, INT8 row; section 2.1]
//   FP8 weight-only  y = bf16(ws[n] * sum_k fp8(w) * x)        [FP8 row; 2.2]
//   FP8 W8A8         y = bf16((acc * xs[m]) * ws[n])           [FP8 row; 2.2]
//   block FP8        y = bf16(sum_kb (D_kb * 2^(ws-127)) * 2^(xs-127))
//                    [Z100 section 2.4: per-block fold; DSV4 section 3.3]
//
// Tiling: a 256-lane workgroup owns a (32*TN weight rows n) x (32*TM tokens
// m) output tile; its 4 waves split it 2 x 2, each wave TN x TM MFMA tiles of
// 16 x 16 (A operand = weight rows, B operand = token rows, so a lane's 4
// accumulator registers are 4 consecutive n of one token).  K runs in tiles
// of BK elements, double-buffered through LDS: the global loads of
// tile k+1 (16 bytes per lane per load, row-contiguous) are in flight while
// tile k is multiplied, then stored to the other LDS buffer; one barrier per
// K tile; whole K tiles are loaded without bounds checks.  (Measured: the
// 32 x 32 MFMAs, deeper prefetch and other LDS paddings do not change the
// throughput of this design; it is bound by the tile traffic through LDS.)  FP8 codes are widened to bf16 (exact) as fragments are read from
// LDS and multiplied on the bf16 matrix core with fp32 accumulation (the
// fp8 matrix-core instructions sum with ~13 bits, see the decode kernels);
// INT8 uses v_mfma_i32_16x16x64_i8 (exact).
//
// Rows past M or N are loaded clamped (results not stored); K chunks past K
// are zero-filled (K % 16 == 0 keeps every 16-byte chunk whole).  Workgroup
// ids are remapped so that each XCD (ids are dealt to the 8 XCDs round
// robin) runs a contiguous range of tiles, M-fastest, so the workgroups
// that share a weight tile share that XCD's L2.
#pragma once
#include <type_traits>

#include "mfma_kernels.hpp"

namespace qlin {

enum GemmAct { kActBf16 = 0, kActE4M3 = 1, kActE5M2 = 2, kActI8 = 3 };
// kEpiBlkG*: block FP8 at any block shape; the suffix is how a row's scale
// bytes of one K tile are fetched (a byte per 32-K step, one 32-bit word for
// block_k 32, one 16-bit half for block_k 64, one byte per tile for block_k
// a multiple of 128)
enum GemmEpi { kEpiI8 = 0, kEpiWs = 1, kEpiXsWs = 2, kEpiBlk = 3, kEpiBlkG = 4, kEpiBlkGW = 5, kEpiBlkGH = 6,
               kEpiBlkGT = 7 };

struct GemmParams {
    const void* x; int64_t ldx;          // activations [M][ldx]: bf16, FP8 or int8 codes
    const float* xs; int xs_step;        // INT8 / W8A8: activation scale [M] or [1]
    const uint8_t* xsb;                  // block FP8: UE8M0 [M][K/128]
    int64_t M, K;
    const void* w; int64_t ldw; int64_t N;  // weight codes [N][ldw]
    const float* ws; int ws_step;        // weight scale [N] or [1]
    const uint8_t* wsb;                  // block FP8: UE8M0 [ceil(N/128)][K/128]
    const uint16_t* bias;                // INT8: bf16 [N] or null
    void* y; int64_t ldy; int out_kind;  // bf16 [M][ldy] (INT8 out_kind 1: int32 acc)
    int64_t bn = 128, bk = 128;          // block FP8, any shape: scale blocks (wsb [ceil(N/bn)][K/bk], xsb [M][K/bk])
};


// 8 FP8 codes (one uint2) of format F -> bf16x8, exact.
template <int F>
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint2 c) {
    bf16x2_t b[4];
    fp8x4_to_bf16<F>(c.x, b[0], b[1]);
    fp8x4_to_bf16<F>(c.y, b[2], b[3]);
    return bf16x8_t{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
}

// Tile shape: a wave computes TN x TM MFMA tiles (16 x 16 each), the 4 waves
// of a workgroup 2 x 2 of those; K tiles of BK elements.
template <int TN, int TM, int BK>
struct GemmShape {
    static constexpr int BN = 32 * TN, BM = 32 * TM;
};

template <int WF, int ACT, int EPI, int TN, int TM, int BK, int PAD = 16>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
    constexpr bool kI8 = ACT == kActI8;
    constexpr int kGemmBN = 32 * TN, kGemmBM = 32 * TM, kGemmBK = BK;
    constexpr int XB = ACT == kActBf16 ? 2 : 1;       // bytes per activation element
    constexpr int WP = kGemmBK + PAD;                 // LDS row pitch, weight tile (bytes)
    constexpr int XP = kGemmBK * XB + PAD;            // LDS row pitch, activation tile
    constexpr int WCPR = kGemmBK / 16;                // 16-byte chunks per row
    constexpr int XCPR = kGemmBK * XB / 16;
    constexpr int WTOT = kGemmBN * WCPR, XTOT = kGemmBM * XCPR;  // chunks per tile
    constexpr int WCH = (WTOT + 255) / 256, XCH = (XTOT + 255) / 256;  // per lane
    static_assert(EPI != kEpiBlk || (128 % (16 * TN) == 0 && BK <= 128 && 128 % BK == 0),
                  "block FP8: a wave's rows lie in one 128-row scale block, K tiles divide 128");
    __shared__ __align__(16) uint8_t wt[2][kGemmBN * WP];
    __shared__ __align__(16) uint8_t xt[2][kGemmBM * XP];

    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t tiles_m = (M + kGemmBM - 1) / kGemmBM;
    const int64_t tiles = tiles_m * ((N + kGemmBN - 1) / kGemmBN);
    const int64_t per_xcd = (int64_t)gridDim.x / 8;  // the grid is a multiple of 8
    const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;  // workgroup-uniform
    const int64_t n0 = (t / tiles_m) * kGemmBN, m0 = (t % tiles_m) * kGemmBM;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn = wv & 1, wm = wv >> 1;
    const int li = lane & 15, lg = lane >> 4;

    // global sources of this lane's chunks
    const uint8_t* wsrc[WCH];
    int wdst[WCH], wcol[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        const int c = (tid + i * 256) % WTOT, r = c / WCPR;  // lanes past WTOT repeat a chunk (not stored)
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        wcol[i] = (c % WCPR) * 16;
        wsrc[i] = (const uint8_t*)p.w + n * p.ldw + wcol[i];
        wdst[i] = r * WP + wcol[i];
    }
    const uint8_t* xsrc[XCH];
    int xdst[XCH], xcol[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = (tid + i * 256) % XTOT, r = c / XCPR;
        const int64_t m = m0 + r < M ? m0 + r : M - 1;
        xcol[i] = (c % XCPR) * 16;
        xsrc[i] = (const uint8_t*)p.x + (m * p.ldx) * XB + xcol[i];
        xdst[i] = r * XP + xcol[i];
    }
    const int64_t ktiles = (K + kGemmBK - 1) / kGemmBK;
    const int64_t kfull = K / kGemmBK;  // tiles that lie wholly inside K: loaded without checks
    u32x4_t wreg[WCH], xreg[XCH];
    auto gload = [&](int64_t kt) {
        if (kt < kfull) {
#pragma unroll
            for (int i = 0; i < WCH; ++i) wreg[i] = ld_stream(wsrc[i] + kt * kGemmBK);
#pragma unroll
            for (int i = 0; i < XCH; ++i) xreg[i] = ld16(xsrc[i] + kt * kGemmBK * XB);
            return;
        }
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int64_t kb = kt * kGemmBK + wcol[i];  // byte = element offset
            wreg[i] = kb < K ? ld_stream(wsrc[i] + kt * kGemmBK) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int64_t ke = kt * kGemmBK + xcol[i] / XB;
            xreg[i] = ke < K ? ld16(xsrc[i] + kt * kGemmBK * XB) : u32x4_t{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int b) {
#pragma unroll
        for (int i = 0; i < WCH; ++i)
            if (WTOT % 256 == 0 || tid + i * 256 < WTOT) *(u32x4_t*)(wt[b] + wdst[i]) = wreg[i];
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            if (XTOT % 256 == 0 || tid + i * 256 < XTOT) *(u32x4_t*)(xt[b] + xdst[i]) = xreg[i];
    };

    typedef typename std::conditional<kI8, i32x4_t, f32x4_t>::type acc_t;
    acc_t acc[TN][TM], dblk[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            acc[i][j] = acc_t{0, 0, 0, 0};
            dblk[i][j] = acc_t{0, 0, 0, 0};
        }
    (void)dblk;

    const int64_t nkb = K >> 7;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int b = (int)(kt & 1);
        if (kt + 1 < ktiles) gload(kt + 1);
        const uint8_t* W = wt[b] + (wn * TN * 16 + li) * WP;
        const uint8_t* X = xt[b] + (wm * TM * 16 + li) * XP;
        if constexpr (kI8) {
#pragma unroll
            for (int ks = 0; ks < kGemmBK / 64; ++ks) {
                i32x4_t a[TN], bb[TM];
#pragma unroll
                for (int i = 0; i < TN; ++i) a[i] = *(const i32x4_t*)(W + i * 16 * WP + ks * 64 + lg * 16);
#pragma unroll
                for (int j = 0; j < TM; ++j) bb[j] = *(const i32x4_t*)(X + j * 16 * XP + ks * 64 + lg * 16);
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bb[j], acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kGemmBK / 32; ++ks) {
                bf16x8_t a[TN], bb[TM];
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    a[i] = fp8x8_to_bf16x8<WF>(*(const uint2*)(W + i * 16 * WP + ks * 32 + lg * 8));
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    if constexpr (ACT == kActBf16)
                        bb[j] = *(const bf16x8_t*)(X + j * 16 * XP + ks * 64 + lg * 16);
                    else
                        bb[j] = fp8x8_to_bf16x8<ACT == kActE5M2 ? kFmtE5M2 : kFmtE4M3>(
                            *(const uint2*)(X + j * 16 * XP + ks * 32 + lg * 8));
                }
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        if constexpr (EPI == kEpiBlk)
                            dblk[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], dblk[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
                    }
            }
            if constexpr (EPI == kEpiBlk) {
                if (((kt + 1) * kGemmBK) % 128 == 0) {  // a 128-wide K block is complete: fold its scales
                    const int64_t kb = ((kt + 1) * kGemmBK >> 7) - 1;
                    const float sw = ue8m0_to_f32(p.wsb[((n0 + wn * TN * 16) >> 7) * nkb + kb]);
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        const int64_t m = m0 + wm * TM * 16 + j * 16 + li;
                        const float sx = ue8m0_to_f32(p.xsb[(m < M ? m : M - 1) * nkb + kb]);
#pragma unroll
                        for (int i = 0; i < TN; ++i) {
                            acc[i][j] += (dblk[i][j] * sx) * sw;
                            dblk[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                }
            }
        }
        if (kt + 1 < ktiles) lstore(b ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds D[n = 4*lg + r][m = li] of each 16 x 16 tile
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int64_t m = m0 + wm * TM * 16 + j * 16 + li;
        if (m >= M) continue;
        float xsv = 1.0f;
        if constexpr (EPI == kEpiI8 || EPI == kEpiXsWs) xsv = p.xs[m * p.xs_step];
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = n0 + wn * TN * 16 + i * 16 + 4 * lg + r;
                if (n >= N) continue;
                if constexpr (EPI == kEpiI8) {
                    if (p.out_kind == 1) {
                        ((int32_t*)p.y)[m * p.ldy + n] = acc[i][j][r];
                        continue;
                    }
                    float v = (float)acc[i][j][r];
                    v = v * xsv;
                    v = v * p.ws[n * p.ws_step];
                    uint16_t o = f32_to_bf16(v);
                    if (p.bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(p.bias[n]));
                    ((uint16_t*)p.y)[m * p.ldy + n] = o;
                } else if constexpr (EPI == kEpiWs) {
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(acc[i][j][r] * p.ws[n * p.ws_step]);
                } else if constexpr (EPI == kEpiXsWs) {
                    float v = acc[i][j][r] * xsv;
                    v = v * p.ws[n * p.ws_step];
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(v);
                } else {
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(acc[i][j][r]);
                }
            }
    }
}

// ------------------------------------------------------------------ direct-to-LDS variant
// For one-byte weight codes and K a multiple of 128 (INT8, FP8 weight-only
// with bf16 activations, FP8 W8A8, block FP8).  The tiles travel global -> LDS with
// global_load_lds_dwordx4 (no VGPR staging, no LDS store instructions) into a
// two-stage ring of 128-byte-deep K tiles: one load instruction covers 8 rows
// x 128 bytes, i.e. whole 128-byte lines (64-byte row pieces measured 40%
// slower through L2).  In LDS a row's 16-byte chunk c sits at position
// c ^ ((row >> 1) & 7), so the 32x32 MFMA fragment reads (16 bytes of 32
// consecutive rows per half-wave) spread over all banks; a lane picks the
// global chunk that lands on its fixed LDS slot.  Each wave waits for its own
// loads with an explicit vmcnt, then one barrier publishes the stage to the
// workgroup (a __syncthreads() would make the compiler drain every
// outstanding load first).  NW = 4 or 8 waves, (NW/2) x 2, each
// (BN/(NW/2)) x (BM/2) of 32 x 32
// MFMA tiles: v_mfma_i32_32x32x32_i8 for INT8; FP8 codes are widened to bf16
// as fragments are read (exact) for v_mfma_f32_32x32x16_bf16.  The block-FP8
// epilogue folds both scales per K tile (= one 128-wide K block).
// Measured at N = 17408, K = 5120 (INT8): M = 128 / 512 / 2048 / 4096 about
// 8 / 20 / 11 / 10% faster than gemm_kernel.  The kernel is bound by the
// tile loads (with the matrix-core work taken out it runs within 3% of the
// full kernel at M = 2048), so the choices below are about feeding it:
// 8 waves on a 128 x 128 tile (two workgroups, 16 waves per compute unit)
// beat 4 (355 -> 310 us at M = 2048; on the 64 x 128 tile at M = 512,
// 112.6 -> 109.0 us), and a banded tile order (below)
// trims L2 misses (310 -> 302 us); deeper LDS rings (3-5 stages, one
// workgroup per unit), 256 x 256 / 256 x 128 tiles (4, 8 or 16 waves) and
// a per-workgroup rotation of the K order were all slower (340-460 us).
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int N_>
__device__ __forceinline__ void wait_vmcnt() {  // s_waitcnt vmcnt(N_), other counters untouched
    static_assert(N_ >= 0 && N_ < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier that does not wait for outstanding global loads: the
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void stage_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int dma_swz(int row) { return (row >> 1) & 7; }

// 8 E4M3 codes times a power-of-two scale -> bf16x8 (the scale is applied
// inside the convert; exact while the results stay in bf16's normal range).
__device__ __forceinline__ bf16x8_t e4m3x8_scaled(uint2 c, float sc) {
    const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false);
    const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true);
    const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false);
    const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true);
    return bf16x8_t{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
}
// activation rows: 8 chunks (one-byte codes, as the weights) or 16 (bf16:
// 32 lanes read one chunk of 32 consecutive rows; chunk ^ (row & 15) spreads
// every 16 of them over all banks)
template <int XB>
__device__ __forceinline__ int dma_xswz(int row) { return XB == 2 ? (row & 15) : dma_swz(row); }

constexpr int64_t kBandM = 8;  // token tiles per raster band (measured at 2048 x 17408 x 5120: 8 > 4 > 2 > none)

template <int WF, int ACT, int EPI, int BN, int BM, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_dma_kernel(const GemmParams p) {
    constexpr bool kI8 = ACT == kActI8;
    static_assert(NW == 4 || NW == 8, "waves");
    // wave grid (weight rows x tokens): two token columns, or four when 8
    // waves share a 64-row tile
    constexpr int WGM = (NW == 8 && BN < 128) ? 4 : 2, WGN = NW / WGM;
    static_assert(BN % (32 * WGN) == 0 && BM % (32 * WGM) == 0 && BN <= 32 * WGN * 2 && BM <= 128, "tile");
    constexpr int BK = 128;                                // K elements per stage (= weight bytes per row)
    constexpr int XB = ACT == kActBf16 ? 2 : 1;            // bytes per activation element
    constexpr int XRB = BK * XB, XRPI = 1024 / XRB;        // activation row bytes, rows per load instruction
    constexpr int WT = BN * BK, XT = BM * XRB, ST = WT + XT;
    constexpr int WI = BN / 8 / NW, XI = BM / XRPI / NW;   // load instructions per wave and stage
    static_assert(WI >= 1 && XI >= 1, "load split");
    constexpr int TN = BN / WGN / 32, TM = BM / WGM / 32;  // 32 x 32 tiles per wave
    __shared__ __align__(16) uint8_t lds[2 * ST];

    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tiles = tiles_m * ((N + BN - 1) / BN);
    const int64_t per_xcd = (int64_t)gridDim.x / 8;  // the grid is a multiple of 8
    const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;  // workgroup-uniform
    // bands of kBandM token tiles: the tile order runs over all weight-row
    // tiles of one band before the next band, so the workgroups that run at
    // once on an XCD share about as many activation tiles as weight tiles
    const int64_t tiles_n = (N + BN - 1) / BN, bsz = kBandM * tiles_n, band = t / bsz, rr = t - band * bsz;
    const int64_t gm = tiles_m - band * kBandM < kBandM ? tiles_m - band * kBandM : kBandM;
    const int64_t n0 = (rr / gm) * BN, m0 = (band * kBandM + rr % gm) * BM;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    // this lane's load sources: row (wv*WI + i)*8 + lane/8, the chunk that
    // belongs in LDS slot lane%8 of that row
    const uint8_t* wsrc[WI];
    const uint8_t* xsrc[XI];
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int r = (wv * WI + i) * 8 + (lane >> 3);
        const int64_t n = n0 + r < N ? n0 + r : N - 1;  // rows past N: clamped, not stored
        wsrc[i] = (const uint8_t*)p.w + n * p.ldw + (((lane & 7) ^ dma_swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = (wv * XI + i) * XRPI + lane / (XRB / 16);
        const int64_t m = m0 + r < M ? m0 + r : M - 1;
        xsrc[i] = (const uint8_t*)p.x + m * p.ldx * XB + (((lane % (XRB / 16)) ^ dma_xswz<XB>(r)) * 16);
    }
    auto issue = [&](int64_t kt, int slot) {
        uint8_t* base = lds + slot * ST;
#pragma unroll
        for (int i = 0; i < WI; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + kt * BK),
                                             (lds_void_t*)(base + (wv * WI + i) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < XI; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xsrc[i] + kt * XRB),
                                             (lds_void_t*)(base + WT + (wv * XI + i) * 1024), 16, 0, 0);
    };

    const int wn = wv % WGN, wm = wv / WGN;
    const int row = lane & 31, half = lane >> 5;
    typedef typename std::conditional<kI8, i32x16_t, f32x16_t>::type acc_t;
    acc_t acc[TN][TM], dblk[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            acc[i][j] = acc_t{};
            dblk[i][j] = acc_t{};
        }
    (void)dblk;

    constexpr bool kBG = EPI >= kEpiBlkG;  // block FP8, any shape
    constexpr int GM = EPI - kEpiBlkG;    // scale fetch: 0 bytes, 1 word, 2 half, 3 one byte per tile
    static_assert(!kBG || (ACT == kActE4M3 && WF == kFmtE4M3), "block FP8 codes");
    const int64_t ktiles = K / BK, nkb = K >> 7;
    // block FP8 at any block shape: a lane's A row and B token are fixed, so
    // each 32-K step needs one weight scale per row tile and one activation
    // scale per token tile; they are folded into the E4M3 -> bf16 converts
    // (exact while the scaled values stay in bf16's normal range) and the
    // products accumulate straight into fp32.  The scale bytes of the next
    // K tile are requested ahead of its loads, as for the 128 x 128 fold.
    constexpr int KSS = BK / 32;  // 32-K steps per tile
    uint32_t gswb[TN][KSS], gsxb[TM][KSS];
    const uint8_t* gsw_row[TN];
    const uint8_t* gsx_row[TM];
    (void)gswb;
    (void)gsxb;
    (void)gsw_row;
    (void)gsx_row;
    if constexpr (kBG) {
        const int64_t nkbg = K / p.bk;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int64_t n = n0 + wn * (BN / WGN) + i * 32 + row;
            gsw_row[i] = p.wsb + ((n < N ? n : N - 1) / p.bn) * nkbg;
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int64_t m = m0 + wm * (BM / WGM) + j * 32 + row;
            gsx_row[j] = p.xsb + (m < M ? m : M - 1) * nkbg;
        }
    }
    // block_k 32 / 64 (GM 1 / 2): a row's scale bytes of one K tile are
    // contiguous (4 / 2 bytes at an aligned offset, K % 128 == 0), so one
    // load per row replaces 4 byte loads, each of which touches 32 rows'
    // cache lines; other block_k load a byte per 32-K step (GM 0).  Words are
    // split at the top of the next step.
    auto load_gscales = [&](int64_t kt) {
        if constexpr (kBG && GM == 1) {
#pragma unroll
            for (int i = 0; i < TN; ++i) gswb[i][0] = *(const uint32_t*)(gsw_row[i] + kt * 4);
#pragma unroll
            for (int j = 0; j < TM; ++j) gsxb[j][0] = *(const uint32_t*)(gsx_row[j] + kt * 4);
        } else if constexpr (kBG && GM == 2) {
#pragma unroll
            for (int i = 0; i < TN; ++i) gswb[i][0] = *(const uint16_t*)(gsw_row[i] + kt * 2);
#pragma unroll
            for (int j = 0; j < TM; ++j) gsxb[j][0] = *(const uint16_t*)(gsx_row[j] + kt * 2);
        } else if constexpr (kBG && GM == 3) {
            const int kb = (int)(kt * BK / p.bk);
#pragma unroll
            for (int i = 0; i < TN; ++i) gswb[i][0] = gsw_row[i][kb];
#pragma unroll
            for (int j = 0; j < TM; ++j) gsxb[j][0] = gsx_row[j][kb];
        } else if constexpr (kBG) {
#pragma unroll
            for (int ks = 0; ks < KSS; ++ks) {
                const int kb = (int)((kt * BK + ks * 32) / p.bk);
#pragma unroll
                for (int i = 0; i < TN; ++i) gswb[i][ks] = gsw_row[i][kb];
#pragma unroll
                for (int j = 0; j < TM; ++j) gsxb[j][ks] = gsx_row[j][kb];
            }
        }
    };
    // scale byte of 32-K step ks from what load_gscales fetched
    auto gbyte = [&](const uint32_t (&v)[KSS], int ks) -> uint32_t {
        if constexpr (GM == 1) return (v[0] >> (8 * ks)) & 0xFFu;
        else if constexpr (GM == 2) return (v[0] >> (8 * (ks >> 1))) & 0xFFu;
        else if constexpr (GM == 3) return v[0];
        else return v[ks];
    };
    (void)gbyte;
    // block FP8: the scale bytes of K block kb are requested one tile ahead,
    // together with that tile, so the wait at the top of the loop covers them
    uint32_t swb = 0, sxb[TM];
    auto load_scales = [&](int64_t kb) {
        if constexpr (EPI == kEpiBlk) {
            swb = p.wsb[(n0 >> 7) * nkb + kb];
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int64_t m = m0 + wm * (BM / WGM) + j * 32 + row;
                sxb[j] = p.xsb[(m < M ? m : M - 1) * nkb + kb];
            }
        }
    };
    load_scales(0);
    load_gscales(0);
    issue(0, 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        wait_vmcnt<0>();  // this wave's loads of tile kt (and its scales), the only ones outstanding
        stage_barrier();  // tile kt complete for everyone; everyone is done with tile kt-1
        float sw = 1.0f, sx[TM];
        if constexpr (EPI == kEpiBlk) {
            // decoded here, before the next bytes are requested: the empty asm
            // pins the value, so the compiler cannot sink the decode to the fold
            // (that would keep the byte register live across its reload and
            // make it wait for every outstanding load)
            sw = ue8m0_to_f32(swb);
            asm volatile("" : "+v"(sw));
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                sx[j] = ue8m0_to_f32(sxb[j]);
                asm volatile("" : "+v"(sx[j]));
            }
        }
        (void)sw;
        (void)sx;
        float gsw[TN][KSS], gsx[TM][KSS];
        (void)gsw;
        (void)gsx;
        if constexpr (kBG) {
#pragma unroll
            for (int ks = 0; ks < KSS; ++ks) {
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    gsw[i][ks] = ue8m0_to_f32(gbyte(gswb[i], ks));
                    asm volatile("" : "+v"(gsw[i][ks]));
                }
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    gsx[j][ks] = ue8m0_to_f32(gbyte(gsxb[j], ks));
                    asm volatile("" : "+v"(gsx[j][ks]));
                }
            }
        }
        load_scales(kt + 1 < ktiles ? kt + 1 : kt);
        load_gscales(kt + 1 < ktiles ? kt + 1 : kt);
        __builtin_amdgcn_sched_barrier(0);  // the scale loads stay ahead of the tile loads
        // unconditional, so the scale loads above complete before it on every
        // path (a conditional issue makes the compiler wait for everything);
        // the last tile reloads itself into the idle slot
        issue(kt + 1 < ktiles ? kt + 1 : kt, (int)((kt + 1) & 1));
        const uint8_t* Wt = lds + (kt & 1) * ST;
        const uint8_t* Xt = Wt + WT;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int c = 2 * ks + half;
            u32x4_t a[TN], b[TM][XB];
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int r = wn * (BN / WGN) + i * 32 + row;
                a[i] = *(const u32x4_t*)(Wt + r * BK + ((c ^ dma_swz(r)) * 16));
            }
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int r = wm * (BM / WGM) + j * 32 + row;
#pragma unroll
                for (int h = 0; h < XB; ++h)  // bf16: the two chunks of the same 16 K
                    b[j][h] = *(const u32x4_t*)(Xt + r * XRB + (((XB * c + h) ^ dma_xswz<XB>(r)) * 16));
            }
            if constexpr (kI8) {
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a[i]),
                                                                         __builtin_bit_cast(i32x4_t, b[j][0]),
                                                                         acc[i][j], 0, 0, 0);
            } else {
                constexpr int XF = ACT == kActE5M2 ? kFmtE5M2 : kFmtE4M3;
                bf16x8_t a0[TN], a1[TN], b0[TM], b1[TM];
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    if constexpr (kBG) {
                        a0[i] = e4m3x8_scaled(make_uint2(a[i].x, a[i].y), gsw[i][ks]);
                        a1[i] = e4m3x8_scaled(make_uint2(a[i].z, a[i].w), gsw[i][ks]);
                    } else {
                        a0[i] = fp8x8_to_bf16x8<WF>(make_uint2(a[i].x, a[i].y));
                        a1[i] = fp8x8_to_bf16x8<WF>(make_uint2(a[i].z, a[i].w));
                    }
                }
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    if constexpr (XB == 2) {
                        b0[j] = __builtin_bit_cast(bf16x8_t, b[j][0]);
                        b1[j] = __builtin_bit_cast(bf16x8_t, b[j][XB - 1]);
                    } else if constexpr (kBG) {
                        b0[j] = e4m3x8_scaled(make_uint2(b[j][0].x, b[j][0].y), gsx[j][ks]);
                        b1[j] = e4m3x8_scaled(make_uint2(b[j][0].z, b[j][0].w), gsx[j][ks]);
                    } else {
                        b0[j] = fp8x8_to_bf16x8<XF>(make_uint2(b[j][0].x, b[j][0].y));
                        b1[j] = fp8x8_to_bf16x8<XF>(make_uint2(b[j][0].z, b[j][0].w));
                    }
                }
#pragma unroll
                for (int i = 0; i < TN; ++i)
#pragma unroll
                    for (int j = 0; j < TM; ++j) {
                        acc_t& d = EPI == kEpiBlk ? dblk[i][j] : acc[i][j];
                        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], d, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], d, 0, 0, 0);
                    }
            }
        }
        if constexpr (EPI == kEpiBlk) {  // the tile is one 128-wide K block: fold its scales
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    acc[i][j] += (dblk[i][j] * sx[j]) * sw;
                    dblk[i][j] = acc_t{};
                }
        }
    }

    wait_vmcnt<0>();  // no load into LDS outlives the workgroup

    // epilogue: register r of a 32 x 32 tile holds weight row 8(r/4) + 4*half + r%4, token lane%32
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int64_t m = m0 + wm * (BM / WGM) + j * 32 + row;
        if (m >= M) continue;
        float xsv = 1.0f;
        if constexpr (EPI == kEpiI8 || EPI == kEpiXsWs) xsv = p.xs[m * p.xs_step];
        (void)xsv;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t n = n0 + wn * (BN / WGN) + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (n >= N) continue;
                if constexpr (EPI == kEpiI8) {
                    if (p.out_kind == 1) {
                        ((int32_t*)p.y)[m * p.ldy + n] = acc[i][j][r];
                        continue;
                    }
                    float v = (float)acc[i][j][r];
                    v = v * xsv;
                    v = v * p.ws[n * p.ws_step];
                    uint16_t o = f32_to_bf16(v);
                    if (p.bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(p.bias[n]));
                    ((uint16_t*)p.y)[m * p.ldy + n] = o;
                } else if constexpr (EPI == kEpiXsWs) {
                    float v = acc[i][j][r] * xsv;
                    v = v * p.ws[n * p.ws_step];
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(v);
                } else if constexpr (EPI == kEpiWs) {
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(acc[i][j][r] * p.ws[n * p.ws_step]);
                } else {
                    ((uint16_t*)p.y)[m * p.ldy + n] = f32_to_bf16(acc[i][j][r]);
                }
            }
    }
}

}  // namespace qlin
