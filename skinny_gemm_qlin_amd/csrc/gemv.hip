// gemv.hip -- launchers of the skinny-GEMV kernels (VALU templates in
// gemv_kernels.hpp, matrix-core templates in mfma_kernels.hpp) with the
// per-M choice of kernel and tile, made by measurement on MI355X at the
// decode shapes (N=17408, K=5120 for INT8 / E4M3; N=4096, K=7168 for block
// FP8):
//   * M = 1: VALU, one whole wavefront per row (GS=64), all K steps of the
//     row in flight (up to 8, or 16 with the token row in LDS); INT8 with 4
//     waves per workgroup (the codes-in-LDS kernel above 8 steps), the FP8
//     kinds (weight-only and W8A8) with the token row staged once per
//     8-wave workgroup in LDS as bf16; block FP8 uses its own M = 1 kernel
//     that shares the scale bytes of a batch across the wave;
//   * M = 2 (INT8 also M = 3): E4M3 weight-only (K <= 16384) one wave per
//     row with both token rows in LDS; INT8 (K <= 16384) one wave per row
//     with the codes in LDS; FP8 W8A8 (K <= 8192) VALU with 32-lane groups
//     of two rows; longer rows as described at each launcher;
//   * K a multiple of 1024 (at most 14336 for INT8, 8192 for the E4M3
//     kinds; see each launcher for the token counts), from M = 4 for INT8
//     and M = 3 for the E4M3 kinds (W8A8 in all four format pairs): the K-slice
//     matrix-core kernels of ks_kernels.hpp, planned here (ks_plan) and
//     launched from ks_i8.hip / ks_f8.hip / ks_w8a8_*.hip (INT8 at M = 4 / 8 /
//     16: 16.4 / 16.8 / 17.3 us against 17.5 / 19.1 / 21.4 us for one
//     workgroup per 16-row tile);
//   * otherwise: the matrix-core kernels of mfma_kernels.hpp;
//   * M > 16 (prefill): the tiled matrix-core GEMM of gemm.hip; on a matrix
//     too small to give the chip enough 64 x 64 tiles, the matrix-core
//     kernels above over a grid of 16-token blocks (split-K inside each
//     workgroup).
#include <algorithm>
#include <atomic>

#include "gemv_kernels.hpp"
#include "ks_launch.hpp"
#include "mfma_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

constexpr int64_t kDecodeMaxM = 16;  // the decode kernels serve M <= 16, the tiled GEMM the rest

namespace {

template <int M, int GS, int R, int U, int WPB>
hipError_t run_i8(const I8Args& a, hipStream_t st) {
    constexpr int rows_per_block = (64 / GS) * R * WPB;
    dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((gemv_i8_kernel<M, GS, R, U, WPB>), grid, dim3(64 * WPB), 0, st,
                       a.xq, a.ldxq, a.xs, a.xs_step, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step,
                       a.bias, a.y, a.ldy, a.out_kind);
    return hipGetLastError();
}

template <int M, int GS, int R, int U, int WPB, int XF, int WF>
hipError_t run_w8a8_fmt(const W8A8F8Args& a, hipStream_t st) {
    constexpr int rows_per_block = (64 / GS) * R * WPB;
    dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((gemv_fp8_w8a8_kernel<M, GS, R, U, WPB, XF, WF>), grid, dim3(64 * WPB), 0, st,
                       a.xq, a.ldxq, a.xs, a.xs_step, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
    return hipGetLastError();
}

// The two code formats are template arguments (the convert instruction
// differs); the four combinations share every tile choice.
template <int M, int GS, int R, int U, int WPB>
hipError_t run_w8a8(const W8A8F8Args& a, hipStream_t st) {
    if (a.x_fmt == kFmtE5M2)
        return a.w_fmt == kFmtE5M2 ? run_w8a8_fmt<M, GS, R, U, WPB, kFmtE5M2, kFmtE5M2>(a, st)
                                   : run_w8a8_fmt<M, GS, R, U, WPB, kFmtE5M2, kFmtE4M3>(a, st);
    return a.w_fmt == kFmtE5M2 ? run_w8a8_fmt<M, GS, R, U, WPB, kFmtE4M3, kFmtE5M2>(a, st)
                               : run_w8a8_fmt<M, GS, R, U, WPB, kFmtE4M3, kFmtE4M3>(a, st);
}

template <int M, int GS, int R, int U, int WPB>
hipError_t run_blk(const BlkArgs& a, hipStream_t st) {
    constexpr int rows_per_block = (64 / GS) * R * WPB;
    dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((gemv_fp8_blk_kernel<M, GS, R, U, WPB>), grid, dim3(64 * WPB), 0, st,
                       a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.y, a.ldy);
    return hipGetLastError();
}

// Number of K steps (GS chunks of 16 bytes) -> unroll for the one-row-per-wave
// M = 1 kernels: every step of the row in flight when there are at most 8.
inline int steps64(int64_t K) { return (int)(((K >> 4) + 63) / 64); }

#define QLIN_M1_BY_STEPS(RUN, a, st)                                  \
    switch (std::min(steps64((a).K), 8)) {                            \
        case 1: return RUN<1, 64, 1, 1, 4>(a, st);                    \
        case 2: return RUN<1, 64, 1, 2, 4>(a, st);                    \
        case 3: return RUN<1, 64, 1, 3, 4>(a, st);                    \
        case 4: return RUN<1, 64, 1, 4, 4>(a, st);                    \
        case 5: return RUN<1, 64, 1, 5, 4>(a, st);                    \
        case 6: return RUN<1, 64, 1, 6, 4>(a, st);                    \
        case 7: return RUN<1, 64, 1, 7, 4>(a, st);                    \
        default: return RUN<1, 64, 1, 8, 4>(a, st);                   \
    }


// One token, FP8 weights: the activation row staged once per workgroup in LDS
// (gemv_fp8_m1_lds_kernel), K <= 8192 (at most 8 steps of 1 KB per row).
// 8 waves per workgroup (17408 x 5120: 14.6-15.1 us against 15.3-16.1 us for
// the register-only kernel it replaced).
constexpr int kM1LdsWaves = 8;
constexpr int64_t kM1LdsMaxK = 8192;

template <int W8A8, int XF, int WF, int U>
void launch_fp8_m1_lds_u(const void* x, const float* xs, int64_t K, const uint8_t* w, int64_t ldw, int64_t N,
                         const float* ws, int ws_step, uint16_t* y, hipStream_t st) {
    const size_t lds = (size_t)(((K >> 3) + 63) / 64) * 1024;  // whole 1 KB direct-load blocks of 2*K/16 halves
    hipLaunchKernelGGL((gemv_fp8_m1_lds_kernel<W8A8, U, kM1LdsWaves, XF, WF>),
                       dim3((unsigned)((N + kM1LdsWaves - 1) / kM1LdsWaves)), dim3(64 * kM1LdsWaves), lds, st,
                       x, xs, K, w, ldw, N, ws, ws_step, y);
}

template <int W8A8, int XF = kFmtE4M3, int WF = kFmtE4M3>
hipError_t run_fp8_m1_lds(const void* x, const float* xs, int64_t K, const uint8_t* w, int64_t ldw, int64_t N,
                          const float* ws, int ws_step, uint16_t* y, hipStream_t st) {
#define QLIN_M1_LDS(U_) launch_fp8_m1_lds_u<W8A8, XF, WF, U_>(x, xs, K, w, ldw, N, ws, ws_step, y, st); break;
    switch (steps64(K)) {
        case 1: QLIN_M1_LDS(1)
        case 2: QLIN_M1_LDS(2)
        case 3: QLIN_M1_LDS(3)
        case 4: QLIN_M1_LDS(4)
        case 5: QLIN_M1_LDS(5)
        case 6: QLIN_M1_LDS(6)
        case 7: QLIN_M1_LDS(7)
        default: QLIN_M1_LDS(8)
    }
#undef QLIN_M1_LDS
    return hipGetLastError();
}

// E4M3 weight-only, one token, 9 to 16 steps of 1 KB per row (8192 < K <=
// 16384): the same kernel with every step in flight (4096 x 14336: 21.5 us
// on the lane-group kernel before).
constexpr int64_t kM1LdsWideMaxK = 16384;

hipError_t run_fp8_m1_lds_wide(const void* x, int64_t K, const uint8_t* w, int64_t ldw, int64_t N, const float* ws,
                               int ws_step, uint16_t* y, hipStream_t st) {
#define QLIN_M1_LDS(U_) launch_fp8_m1_lds_u<0, kFmtE4M3, kFmtE4M3, U_>(x, nullptr, K, w, ldw, N, ws, ws_step, y, st); break;
    switch (steps64(K)) {
        case 9: QLIN_M1_LDS(9)
        case 10: QLIN_M1_LDS(10)
        case 11: QLIN_M1_LDS(11)
        case 12: QLIN_M1_LDS(12)
        case 13: QLIN_M1_LDS(13)
        case 14: QLIN_M1_LDS(14)
        case 15: QLIN_M1_LDS(15)
        default: QLIN_M1_LDS(16)
    }
#undef QLIN_M1_LDS
    return hipGetLastError();
}

// E4M3 weight-only, two tokens: one wave per row with every 1 KB step in
// flight, the token rows staged once per 8-wave workgroup in LDS as bf16
// (gemv_fp8_lds_kernel), K <= 16384.  Against the K-slice / lane-group
// kernels it replaced at M = 2: 4096 x 14336 15.0 vs 18.5 us, 8192 x 8192
// 14.1 vs 15.9 us, 4096 x 10240 10.8 vs 14.2 us, equal within 0.2 us at
// 17408 x 5120, 14336 x 4096, 28672 x 4096 and 4096 x 4096.  With three or
// four tokens its dot products outweigh the stream (17408 x 5120: 21.6 /
// 25.5 us against 17.2 / 17.3 us for the K-slice kernels), so it stops at two.
constexpr int64_t kF8LdsMaxK = 16384;

template <int M, int U, bool LOOP = false>
void launch_fp8_lds_u(const F8Args& a, hipStream_t st) {
    const size_t lds = (size_t)((M * (a.K >> 3) + 63) / 64) * 1024;
    hipLaunchKernelGGL((gemv_fp8_lds_kernel<M, U, kM1LdsWaves, LOOP>), dim3((unsigned)((a.N + kM1LdsWaves - 1) / kM1LdsWaves)),
                       dim3(64 * kM1LdsWaves), lds, st, a.x, a.ldx, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
}

template <int M>
hipError_t run_fp8_lds(const F8Args& a, hipStream_t st) {
#define QLIN_F8_LDS(U_) launch_fp8_lds_u<M, U_>(a, st); break;
    switch (steps64(a.K)) {
        case 1: QLIN_F8_LDS(1)
        case 2: QLIN_F8_LDS(2)
        case 3: QLIN_F8_LDS(3)
        case 4: QLIN_F8_LDS(4)
        case 5: QLIN_F8_LDS(5)
        case 6: QLIN_F8_LDS(6)
        case 7: QLIN_F8_LDS(7)
        case 8: QLIN_F8_LDS(8)
        case 9: QLIN_F8_LDS(9)
        case 10: QLIN_F8_LDS(10)
        case 11: QLIN_F8_LDS(11)
        case 12: QLIN_F8_LDS(12)
        case 13: QLIN_F8_LDS(13)
        case 14: QLIN_F8_LDS(14)
        case 15: QLIN_F8_LDS(15)
        default: QLIN_F8_LDS(16)
    }
#undef QLIN_F8_LDS
    return hipGetLastError();
}

// One token with rows of more than 16 steps on a matrix with fewer than 4096
// rows: the same kernel taking 16 steps of the row at a time, the bf16 row in
// LDS up to 64 KB (K <= 32768); 2048 x 32768: 17.0 against 22.7 us for the
// per-tile matrix-core kernel, which is faster from 4096 rows (4096 x 20480:
// 17.4 against 25.6 us).
constexpr int64_t kF8LdsLoopMaxK = 32768;

hipError_t run_fp8_lds_loop(const F8Args& a, hipStream_t st) {
    launch_fp8_lds_u<1, 16, true>(a, st);
    return hipGetLastError();
}

// INT8, 2..3 tokens (and one token with the quantiser fused in): one wave
// per row, the token rows' codes shared through LDS (gemv_i8_lds_kernel).
// 17408 x 5120: M = 2 14.9-15.1 us against 15.7-16.1 us for the lane-group
// kernel, M = 3 15.8-16.2 us; the fused one-token call 16.2-16.5 us against
// 16.9-17.3 us for quantiser + GEMV in two launches.
constexpr int64_t kI8LdsMaxM = 3;

template <int M, int WPB, bool QX, int U, bool LOOP = false>
void launch_i8_lds_u(const void* x, int64_t ldx, const I8Args& a, int8_t* xq_out, int64_t ldxq, float* xs_out,
                     hipStream_t st) {
    const size_t lds = QX ? (size_t)(M * a.K) : (size_t)((M * (a.K >> 4) + 63) / 64) * 1024;
    hipLaunchKernelGGL((gemv_i8_lds_kernel<M, U, WPB, QX, LOOP>), dim3((unsigned)((a.N + WPB - 1) / WPB)), dim3(64 * WPB),
                       lds, st, x, ldx, a.xs, a.xs_step, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy,
                       a.out_kind, xq_out, ldxq, xs_out);
}

template <int M, int WPB, bool QX>
hipError_t run_i8_lds(const void* x, int64_t ldx, const I8Args& a, int8_t* xq_out, int64_t ldxq, float* xs_out,
                      hipStream_t st) {
#define QLIN_I8_LDS(U_) launch_i8_lds_u<M, WPB, QX, U_>(x, ldx, a, xq_out, ldxq, xs_out, st); break;
    switch (steps64(a.K)) {
        case 1: QLIN_I8_LDS(1)
        case 2: QLIN_I8_LDS(2)
        case 3: QLIN_I8_LDS(3)
        case 4: QLIN_I8_LDS(4)
        case 5: QLIN_I8_LDS(5)
        case 6: QLIN_I8_LDS(6)
        case 7: QLIN_I8_LDS(7)
        default: QLIN_I8_LDS(8)
    }
#undef QLIN_I8_LDS
    return hipGetLastError();
}

// One to three tokens with 9 to 16 steps of 1 KB per row (8192 < K <=
// 16384): the same kernel, every step of the row in flight (4096 x 14336,
// M = 2: 13.7 -> 11.4 us against the lane-group kernel).
constexpr int64_t kI8LdsWideMaxK = 16384;

template <int M>
hipError_t run_i8_lds_wide(const I8Args& a, hipStream_t st) {
#define QLIN_I8_LDS(U_) launch_i8_lds_u<M, 4, false, U_>(a.xq, a.ldxq, a, nullptr, 0, nullptr, st); break;
    switch (steps64(a.K)) {
        case 9: QLIN_I8_LDS(9)
        case 10: QLIN_I8_LDS(10)
        case 11: QLIN_I8_LDS(11)
        case 12: QLIN_I8_LDS(12)
        case 13: QLIN_I8_LDS(13)
        case 14: QLIN_I8_LDS(14)
        case 15: QLIN_I8_LDS(15)
        default: QLIN_I8_LDS(16)
    }
#undef QLIN_I8_LDS
    return hipGetLastError();
}

// Two or three tokens with rows of more than 16 steps (K > 16384) on a matrix
// with fewer than 4096 rows: the same kernel taking 16 steps of the row at a
// time, while the codes fit in 64 KB of LDS.  There the per-tile matrix-core
// kernel has fewer tiles than the chip has compute units (2048 x 32768, M =
// 2: 16.4 against 21.5 us); from 4096 rows it is the faster one (4096 x
// 20480: 16.9 against 24.3 us, 8192 x 28672: 38.6 against 52.0 us).
constexpr int64_t kI8LdsLoopMaxBytes = 64 << 10;
constexpr int64_t kLdsLoopMaxN = 4095;

template <int M>
hipError_t run_i8_lds_loop(const I8Args& a, hipStream_t st) {
    launch_i8_lds_u<M, 4, false, 16, true>(a.xq, a.ldxq, a, nullptr, 0, nullptr, st);
    return hipGetLastError();
}

// Matrix-core kernels: one workgroup of KS waves per 16-row tile, one chunk
// of 256 K per wave per batch (few registers, so the whole grid is resident
// and waves overlap each other's latency; measured at the decode shapes).
// KS splits K so that the grid holds about 4096 waves: 4 when there are at
// least 1024 row tiles, 8 from 512, else 16 -- never more waves than K has
// chunks for, beyond the minimum of 4.
// From 12 tokens the INT8 kernel stages the activation rows through LDS like
// the weights (row-contiguous loads; measured 23.9 -> 22.4 us at M = 16,
// slower below 12 tokens).
constexpr int64_t kStageXMinM = 12;

inline int mfma_ks(int64_t N, int64_t K) {
    const int64_t tiles = (N + 15) / 16, nch = (K + 255) >> 8;
    int ks = tiles >= 1024 ? 4 : (tiles >= 512 ? 8 : 16);
    while (ks > 4 && ks / 2 >= nch) ks /= 2;
    return ks;
}

#define QLIN_BY_KS(KERNEL, KS_, GRID, ...)                                                 \
    switch (KS_) {                                                                        \
        case 16: hipLaunchKernelGGL((KERNEL<1, 16>), GRID, dim3(1024), __VA_ARGS__); break;  \
        case 8: hipLaunchKernelGGL((KERNEL<1, 8>), GRID, dim3(512), __VA_ARGS__); break;     \
        default: hipLaunchKernelGGL((KERNEL<1, 4>), GRID, dim3(256), __VA_ARGS__); break;    \
    }

template <int U>
void launch_i8_xl4(const I8Args& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((gemv_i8_mfma_xl_kernel<U, 4>), grid, dim3(256), 0, st, a.xq, a.ldxq, a.xs, a.xs_step,
                       (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind);
}

hipError_t run_i8_mfma(const I8Args& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16));
    if (a.M >= kStageXMinM) {
        const int ks = mfma_ks(a.N, a.K);
        const int64_t per = ((a.K + 255) / 256 + ks - 1) / ks;  // 256-K chunks per wave
        if (ks == 4 && per <= 5) {
            // every chunk of the wave in flight at once (17408 x 5120, M = 16:
            // 22.6 -> 21.5 us; M = 12: 21.1 -> 20.8 us)
            switch (per) {
                case 5: launch_i8_xl4<5>(a, grid, st); break;
                case 4: launch_i8_xl4<4>(a, grid, st); break;
                case 3: launch_i8_xl4<3>(a, grid, st); break;
                case 2: launch_i8_xl4<2>(a, grid, st); break;
                default: launch_i8_xl4<1>(a, grid, st); break;
            }
            return hipGetLastError();
        }
        QLIN_BY_KS(gemv_i8_mfma_xl_kernel, ks, grid, 0, st, a.xq, a.ldxq, a.xs, a.xs_step,
                   (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind)
    } else {
        QLIN_BY_KS(gemv_i8_mfma_kernel, mfma_ks(a.N, a.K), grid, 0, st, a.xq, a.ldxq, a.xs, a.xs_step, (int)a.M,
                   a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind)
    }
    return hipGetLastError();
}

hipError_t run_fp8_mfma(const F8Args& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16));
    QLIN_BY_KS(gemv_fp8_mfma_kernel, mfma_ks(a.N, a.K), grid, 0, st, a.x, a.ldx, (int)a.M, a.K, a.w, a.ldw,
               a.N, a.ws, a.ws_step, a.y, a.ldy)
    return hipGetLastError();
}

hipError_t run_blk_mfma(const BlkArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16));
    QLIN_BY_KS(gemv_fp8_blk_mfma_kernel, mfma_ks(a.N, a.K), grid, 0, st, a.xq, a.xs, (int)a.M, a.K, a.w,
               a.ldw, a.N, a.ws, a.y, a.ldy)
    return hipGetLastError();
}

template <int XF, int WF, bool XL>
hipError_t run_w8a8_mfma_x(const W8A8F8Args& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16));
    switch (mfma_ks(a.N, a.K)) {
        case 16:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 16, XF, WF, XL>), grid, dim3(1024), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
        case 8:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 8, XF, WF, XL>), grid, dim3(512), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
        default:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 4, XF, WF, XL>), grid, dim3(256), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
    }
    return hipGetLastError();
}

// From 8 tokens the activation codes are staged through LDS like the weights
// (measured at 17408 x 5120: M = 16 26.2 -> 23.2 us, M = 12 23.0 -> 22.1 us).
template <int XF, int WF>
hipError_t run_w8a8_mfma_fmt(const W8A8F8Args& a, hipStream_t st) {
    return a.M >= 8 ? run_w8a8_mfma_x<XF, WF, true>(a, st) : run_w8a8_mfma_x<XF, WF, false>(a, st);
}

hipError_t run_w8a8_mfma(const W8A8F8Args& a, hipStream_t st) {
    if (a.x_fmt == kFmtE5M2)
        return a.w_fmt == kFmtE5M2 ? run_w8a8_mfma_fmt<kFmtE5M2, kFmtE5M2>(a, st)
                                   : run_w8a8_mfma_fmt<kFmtE5M2, kFmtE4M3>(a, st);
    return a.w_fmt == kFmtE5M2 ? run_w8a8_mfma_fmt<kFmtE4M3, kFmtE5M2>(a, st)
                               : run_w8a8_mfma_fmt<kFmtE4M3, kFmtE4M3>(a, st);
}

// ---- prefill on a small weight matrix: split-K over the token-block grid
// The tiled GEMM gives each workgroup a 64 x 64 (or larger) output tile and
// walks all of K in it, so a matrix with few rows gets few workgroups (N = 48,
// M = 64: one workgroup on a 256-unit chip).  Below a quarter of the compute
// units' worth of 64 x 64 tiles the matrix-core decode kernels run instead,
// over a grid of 16-row tiles x 16-token blocks, each workgroup splitting K
// between its waves and summing their partial tiles in wave order.
int cu_count();

bool small_gemm(int64_t M, int64_t N) {
    const int64_t tiles64 = ((N + 63) / 64) * ((M + 63) / 64);
    return tiles64 * 4 < cu_count();
}

// waves per workgroup of the token-block grid: about 4096 waves in all
inline int grid_ks(int64_t N, int64_t M, int64_t K) {
    const int64_t wgs = ((N + 15) / 16) * ((M + 15) / 16), nch = (K + 255) >> 8;
    int ks = wgs >= 1024 ? 4 : (wgs >= 512 ? 8 : 16);
    while (ks > 4 && ks / 2 >= nch) ks /= 2;
    return ks;
}

inline dim3 token_block_grid(int64_t N, int64_t M) {
    return dim3((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
}

hipError_t run_i8_split(const I8Args& a, hipStream_t st) {
    QLIN_BY_KS(gemv_i8_mfma_kernel, grid_ks(a.N, a.M, a.K), token_block_grid(a.N, a.M), 0, st, a.xq, a.ldxq,
               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind)
    return hipGetLastError();
}

hipError_t run_fp8_split(const F8Args& a, hipStream_t st) {
    QLIN_BY_KS(gemv_fp8_mfma_kernel, grid_ks(a.N, a.M, a.K), token_block_grid(a.N, a.M), 0, st, a.x, a.ldx,
               (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy)
    return hipGetLastError();
}

template <int XF, int WF>
hipError_t run_w8a8_split_fmt(const W8A8F8Args& a, hipStream_t st) {
    const dim3 grid = token_block_grid(a.N, a.M);
    switch (grid_ks(a.N, a.M, a.K)) {
        case 16:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 16, XF, WF, true>), grid, dim3(1024), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
        case 8:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 8, XF, WF, true>), grid, dim3(512), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
        default:
            hipLaunchKernelGGL((gemv_fp8_w8a8_mfma_kernel<1, 4, XF, WF, true>), grid, dim3(256), 0, st, a.xq, a.ldxq,
                               a.xs, a.xs_step, (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
            break;
    }
    return hipGetLastError();
}

hipError_t run_w8a8_split(const W8A8F8Args& a, hipStream_t st) {
    if (a.x_fmt == kFmtE5M2)
        return a.w_fmt == kFmtE5M2 ? run_w8a8_split_fmt<kFmtE5M2, kFmtE5M2>(a, st)
                                   : run_w8a8_split_fmt<kFmtE5M2, kFmtE4M3>(a, st);
    return a.w_fmt == kFmtE5M2 ? run_w8a8_split_fmt<kFmtE4M3, kFmtE5M2>(a, st)
                               : run_w8a8_split_fmt<kFmtE4M3, kFmtE4M3>(a, st);
}

hipError_t run_blk_split(const BlkArgs& a, hipStream_t st) {
    QLIN_BY_KS(gemv_fp8_blk_mfma_kernel, grid_ks(a.N, a.M, a.K), token_block_grid(a.N, a.M), 0, st, a.xq, a.xs,
               (int)a.M, a.K, a.w, a.ldw, a.N, a.ws, a.y, a.ldy)
    return hipGetLastError();
}

// ---- K-slice kernels: the plan and the launch
// Compute units of the current device (queried once per device).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// K = 1024 * L with L in [2, lmax]; G = one workgroup per compute unit, or
// one per 16 rows when N is small; the ceil(N/4) runs of 4 rows are dealt
// out in turn, R = rows per workgroup (a multiple of 4).  A workgroup with
// more than kKsMaxTiles tiles runs them in npass passes of T tiles (then
// 4 <= T <= kKsMaxTiles), so the grid never exceeds one workgroup per
// compute unit (a second round of workgroups: 28672 x 4096, M = 4..16,
// 27.9-29.2 us against 22.5-26.3 us in two passes).
bool ks_plan(int64_t N, int64_t K, int lmax, KsPlan& p) {
    if (N < 1 || K % 1024 != 0 || K / 1024 < 2 || K / 1024 > lmax) return false;
    const int64_t runs = (N + 3) / 4;
    const int64_t G = std::min<int64_t>(cu_count(), (N + 15) / 16);
    const int64_t R = 4 * ((runs + G - 1) / G);
    const int64_t tiles = (R + 15) / 16;
    const int64_t npass = (tiles + kKsMaxTiles - 1) / kKsMaxTiles;
    p = {(int)(K / 1024), (int)((tiles + npass - 1) / npass), (unsigned)G, R, (int)npass};
    return true;
}

constexpr int kKsMaxLI8 = 14;    // INT8 holds 2L + D * 2L 16-byte registers per lane (D = 3 / 2 / 1 tiles in
                                 // flight up to 6 / 8 / 14 lines)
constexpr int kKsMaxLFloat = 8;  // the float kinds hold 4L + D * 2L (D = 2 / 1 up to 6 / 8 lines)

template <int U>
hipError_t run_blk_m1(const BlkArgs& a, hipStream_t st) {
    constexpr int WPB = 4;
    dim3 grid((unsigned)((a.N + WPB - 1) / WPB));
    hipLaunchKernelGGL((gemv_fp8_blk_m1_kernel<U, WPB>), grid, dim3(64 * WPB), 0, st, a.xq, a.xs, a.K, a.w,
                       a.ldw, a.N, a.ws, a.y);
    return hipGetLastError();
}

// 16 rows per workgroup: every workgroup quantises the whole row, so fewer,
// larger workgroups cut that redundant work (measured at 4096 x 7168: 4 / 8 /
// 16 waves 9.2 / 7.9 / 7.7 us, quantiser + GEMV in two launches 9.0 us).
template <int U>
hipError_t run_blk_m1_fq(const BlkQuantArgs& q, const BlkArgs& a, hipStream_t st) {
    constexpr int WPB = 16;
    dim3 grid((unsigned)((a.N + WPB - 1) / WPB));
    const size_t lds = (size_t)a.K + sizeof(float) * (size_t)(a.K >> 7);
    hipLaunchKernelGGL((gemv_fp8_blk_m1_fq_kernel<U, WPB>), grid, dim3(64 * WPB), lds, st, q.x, a.K, a.w, a.ldw,
                       a.N, a.ws, q.xq, q.xs, a.y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_i8(const I8Args& a, hipStream_t st) {
    if (a.M > kDecodeMaxM) return small_gemm(a.M, a.N) ? run_i8_split(a, st) : launch_gemm_i8(a, st);
    if (a.M >= 2 && a.M <= kI8LdsMaxM && a.K <= kI8LdsMaxK)
        return a.M == 2 ? run_i8_lds<2, 4, false>(a.xq, a.ldxq, a, nullptr, 0, nullptr, st)
                        : run_i8_lds<3, 4, false>(a.xq, a.ldxq, a, nullptr, 0, nullptr, st);
    if (a.M >= 2 && a.M <= kI8LdsMaxM && a.K <= kI8LdsWideMaxK)
        return a.M == 2 ? run_i8_lds_wide<2>(a, st) : run_i8_lds_wide<3>(a, st);
    if (a.M >= 2 && a.M <= kI8LdsMaxM && a.M * a.K <= kI8LdsLoopMaxBytes && a.N <= kLdsLoopMaxN)
        return a.M == 2 ? run_i8_lds_loop<2>(a, st) : run_i8_lds_loop<3>(a, st);
    switch (a.M) {
        case 1:
            // above 8 steps the codes-in-LDS kernel keeps every step in flight
            // (4096 x 10240: the lane-group kernel loops over 8 at a time)
            if (a.K > kI8LdsMaxK && a.K <= kI8LdsWideMaxK) return run_i8_lds_wide<1>(a, st);
            QLIN_M1_BY_STEPS(run_i8, a, st)
        case 2:
            // rows the LDS kernels above do not take (K > 16384 from 4096
            // rows, or codes past 64 KB): the per-tile matrix-core kernel
            // (4096 x 20480: 17.2 against 20.4 us for the lane-group kernel)
            return run_i8_mfma(a, st);
        default: {
            // above 8 lines (one tile in flight) the K-slice kernels serve up
            // to 8 tokens (4096 x 14336: 12.7 against 13.4 us at M = 8, but
            // 15.2 against 14.6 us at M = 16 for the per-tile kernel)
            // except 12 and 13 lines with two or more tiles per workgroup,
            // which run slower than the per-tile kernel (M = 4: 8192 x 12288
            // 26.3 against 19.1 us, 8192 x 13312 22.1 against 19.9 us,
            // 12288 x 12288 29.0 against 26.2 us; the compiler keeps far fewer
            // loads in flight there: 126 VGPRs at 12 lines and two tiles
            // against 164 at 11)
            KsPlan p;
            if (ks_plan(a.N, a.K, a.M <= 8 ? kKsMaxLI8 : 8, p) &&
                !((p.L == 12 || p.L == 13) && (int64_t)p.T * p.npass >= 2)) {
                const KsArgs k{a.xq, a.ldxq, a.xs, a.xs_step, (int)a.M, (const uint8_t*)a.w, a.ldw, a.N, p.R,
                               a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind};
                return launch_ks_i8(k, p, st);
            }
            return run_i8_mfma(a, st);
        }
    }
}

hipError_t launch_linear_i8_fused(const ActQuantI8Args& q, const I8Args& a, hipStream_t st) {
    if (a.M != 1 || a.K > kI8LdsMaxK) return hipErrorInvalidValue;
    return run_i8_lds<1, 8, true>(q.x, q.ldx, a, q.xq, q.ldxq, q.xs, st);
}

hipError_t launch_gemv_fp8(const F8Args& a, hipStream_t st) {
    if (a.M > kDecodeMaxM) return small_gemm(a.M, a.N) ? run_fp8_split(a, st) : launch_gemm_fp8(a, st);
    switch (a.M) {
        case 1:
            if (a.K <= kM1LdsMaxK)
                return run_fp8_m1_lds<0>(a.x, nullptr, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st);
            if (a.K <= kM1LdsWideMaxK)
                return run_fp8_m1_lds_wide(a.x, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st);
            if (a.K <= kF8LdsLoopMaxK && a.N <= kLdsLoopMaxN) return run_fp8_lds_loop(a, st);
            // else the per-tile matrix-core kernel
            return run_fp8_mfma(a, st);
        default: {
            if (a.M == 2 && a.K <= kF8LdsMaxK) return run_fp8_lds<2>(a, st);
            // K-slice kernels from M = 3, up to 8 lines (14336 x 7168:
            // 19.4-22.8 against 21.5-37.2 us for the per-tile kernel), else
            // the per-tile matrix-core kernel (two tokens above K = 16384 too:
            // 4096 x 20480 18.1 against 25.6 us for the lane-group kernel)
            KsPlan p;
            if (ks_plan(a.N, a.K, kKsMaxLFloat, p)) {
                const KsArgs k{a.x, a.ldx, nullptr, 0, (int)a.M, a.w, a.ldw, a.N, p.R,
                               a.ws, a.ws_step, nullptr, a.y, a.ldy, 0};
                return launch_ks_f8(k, p, st);
            }
            return run_fp8_mfma(a, st);
        }
    }
}

// W8A8 FP8 widens both operands (16 converts per 16 code pairs), so the VALU
// kernels keep fewer steps in flight than INT8 (measured at 17408 x 5120:
// M = 1 best with 3 steps of one row per wave, M = 2 with 32-lane groups and
// 5 steps); the matrix-core kernel from M = 3.
hipError_t launch_gemv_fp8_w8a8(const W8A8F8Args& a, hipStream_t st) {
    if (a.M > kDecodeMaxM) return small_gemm(a.M, a.N) ? run_w8a8_split(a, st) : launch_gemm_fp8_w8a8(a, st);
    if (a.M == 1 && a.K <= kM1LdsMaxK) {
        if (a.x_fmt == kFmtE5M2)
            return a.w_fmt == kFmtE5M2
                       ? run_fp8_m1_lds<1, kFmtE5M2, kFmtE5M2>(a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st)
                       : run_fp8_m1_lds<1, kFmtE5M2, kFmtE4M3>(a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st);
        return a.w_fmt == kFmtE5M2
                   ? run_fp8_m1_lds<1, kFmtE4M3, kFmtE5M2>(a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st)
                   : run_fp8_m1_lds<1, kFmtE4M3, kFmtE4M3>(a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, st);
    }
    if (a.M == 1) {
        switch (std::min(steps64(a.K), 3)) {
            case 1: return run_w8a8<1, 64, 1, 1, 4>(a, st);
            case 2: return run_w8a8<1, 64, 1, 2, 4>(a, st);
            default: return run_w8a8<1, 64, 1, 3, 4>(a, st);
        }
    }
    // two rows per lane group share each activation chunk's convert (measured
    // at N=17408, K=5120: 16.4 us against 17.7-18.5 us for one row per group
    // with 2-5 steps in flight); with one step in flight per group that kernel
    // falls behind on longer rows, where two and three tokens take the
    // per-tile matrix-core kernel (4096 x 14336: 22.6 / 27.8 us on the VALU
    // kernels against 12.8 us at M = 4; 7168 x 9216: 17.5 / 20.8 against 16.3)
    if (a.M <= 3 && a.K > kM1LdsMaxK) return run_w8a8_mfma(a, st);
    if (a.M == 2) return run_w8a8<2, 32, 2, 1, 1>(a, st);
    // from three tokens the K-slice kernels where they apply (E4M3 x E4M3,
    // 17408 x 5120: 16.8 against 18.3 us for the VALU kernel below at M = 3);
    // above 5 lines (codes widened in registers, one tile in flight from 7)
    // only where a workgroup has at least 3 tiles of rows, or at M = 3: with
    // two tiles the per-tile matrix-core kernel is faster from M = 4
    // (8192 x 8192: 14.2-15.6 against 17.4-18.2 us; 14336 x 7168, four tiles:
    // 19.3-20.8 against 22.6-26.6 us)
    KsPlan p;
    if (ks_plan(a.N, a.K, kKsMaxLFloat, p) && (p.L <= 5 || a.M == 3 || (int64_t)p.T * p.npass >= 3)) {
        const KsArgs k{a.xq, a.ldxq, a.xs, a.xs_step, (int)a.M, a.w, a.ldw, a.N, p.R,
                       a.ws, a.ws_step, nullptr, a.y, a.ldy, 0};
        return a.x_fmt == kFmtE5M2 ? launch_ks_w8a8_e5m2(k, p, a.w_fmt, st) : launch_ks_w8a8_e4m3(k, p, a.w_fmt, st);
    }
    // three rows per group at three tokens, K <= 8192 (17.8-17.9 us against
    // 19.1-19.3 us for the matrix-core kernel); from four tokens the matrix
    // core wins
    if (a.M == 3) return run_w8a8<3, 32, 3, 1, 1>(a, st);
    return run_w8a8_mfma(a, st);
}

template <bool PAIR>
hipError_t run_blkg(const BlkArgs& a, int64_t bn, int64_t bk, hipStream_t st) {
    const dim3 grid = token_block_grid(a.N, a.M);  // blockIdx.y: 16-token block
    const size_t lds = (size_t)(a.K / bk) * 32;  // transposed weight and token scale tables
    switch (grid_ks(a.N, a.M, a.K)) {
        case 16:
            hipLaunchKernelGGL((gemv_fp8_blkg_mfma_kernel<16, PAIR>), grid, dim3(1024), lds, st, a.xq, a.xs, (int)a.M,
                               a.K, a.w, a.ldw, a.N, a.ws, bn, bk, a.y, a.ldy);
            break;
        case 8:
            hipLaunchKernelGGL((gemv_fp8_blkg_mfma_kernel<8, PAIR>), grid, dim3(512), lds, st, a.xq, a.xs, (int)a.M,
                               a.K, a.w, a.ldw, a.N, a.ws, bn, bk, a.y, a.ldy);
            break;
        default:
            hipLaunchKernelGGL((gemv_fp8_blkg_mfma_kernel<4, PAIR>), grid, dim3(256), lds, st, a.xq, a.xs, (int)a.M,
                               a.K, a.w, a.ldw, a.N, a.ws, bn, bk, a.y, a.ldy);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_fp8_blkg(const BlkArgs& a, int64_t bn, int64_t bk, hipStream_t st) {
    return bk % 64 == 0 ? run_blkg<true>(a, bn, bk, st) : run_blkg<false>(a, bn, bk, st);
}

hipError_t launch_gemv_fp8_blk(const BlkArgs& a, hipStream_t st) {
    if (a.M > kDecodeMaxM) return small_gemm(a.M, a.N) ? run_blk_split(a, st) : launch_gemm_fp8_blk(a, st);
    if (a.M > 1) return run_blk_mfma(a, st);
    switch (std::min(steps64(a.K), 8)) {
        case 1: return run_blk_m1<1>(a, st);
        case 2: return run_blk_m1<2>(a, st);
        case 3: return run_blk_m1<3>(a, st);
        case 4: return run_blk_m1<4>(a, st);
        case 5: return run_blk_m1<5>(a, st);
        case 6: return run_blk_m1<6>(a, st);
        case 7: return run_blk_m1<7>(a, st);
        default: return run_blk_m1<8>(a, st);
    }
}

// Quantiser fused into the GEMV (one launch) for M = 1; the row is staged in
// LDS, so K is capped (kBlkFusedMaxK).  Up to K = 8192 the 8-wave kernel
// that stages decoded values and waits for no weights at its barrier
// (4096 x 7168: 7.1-7.2 us against 7.6-7.8 us for the 16-wave one below).
template <int U>
hipError_t run_blk_m1_lds(const BlkQuantArgs& q, const BlkArgs& a, hipStream_t st) {
    constexpr int WPB = 8;
    const size_t lds = (size_t)a.K * 2 + sizeof(float) * (size_t)(a.K >> 7);
    hipLaunchKernelGGL((gemv_fp8_blk_m1_lds_kernel<U, WPB>), dim3((unsigned)((a.N + WPB - 1) / WPB)),
                       dim3(64 * WPB), lds, st, q.x, a.K, a.w, a.ldw, a.N, a.ws, q.xq, q.xs, a.y);
    return hipGetLastError();
}

hipError_t launch_gemv_fp8_blk_fq(const BlkQuantArgs& q, const BlkArgs& a, hipStream_t st) {
    if (a.M != 1 || a.K > kBlkFusedMaxK) return hipErrorInvalidValue;
    if (a.K <= kBlkM1LdsMaxK) {
        switch (steps64(a.K)) {
            case 1: return run_blk_m1_lds<1>(q, a, st);
            case 2: return run_blk_m1_lds<2>(q, a, st);
            case 3: return run_blk_m1_lds<3>(q, a, st);
            case 4: return run_blk_m1_lds<4>(q, a, st);
            case 5: return run_blk_m1_lds<5>(q, a, st);
            case 6: return run_blk_m1_lds<6>(q, a, st);
            case 7: return run_blk_m1_lds<7>(q, a, st);
            default: return run_blk_m1_lds<8>(q, a, st);
        }
    }
    switch (std::min(steps64(a.K), 8)) {
        case 1: return run_blk_m1_fq<1>(q, a, st);
        case 2: return run_blk_m1_fq<2>(q, a, st);
        case 3: return run_blk_m1_fq<3>(q, a, st);
        case 4: return run_blk_m1_fq<4>(q, a, st);
        case 5: return run_blk_m1_fq<5>(q, a, st);
        case 6: return run_blk_m1_fq<6>(q, a, st);
        case 7: return run_blk_m1_fq<7>(q, a, st);
        default: return run_blk_m1_fq<8>(q, a, st);
    }
}

}  // namespace qlin
