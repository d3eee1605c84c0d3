// gemv.hip -- launchers of the VALU skinny-GEMV kernels (templates in
// gemv_kernels.hpp) with the per-M tile configuration.
//
// Configuration per M (lanes per row GS, rows per group R, unrolled steps U,
// waves per workgroup WPB) was chosen by measurement on MI355X at the decode
// shapes (N=17408, K=5120 for INT8 / E4M3; N=4096, K=7168 for block FP8):
//   * M = 1: one whole wavefront per row (GS=64), all K steps of the row in
//     flight (U = number of steps, up to 8), 4 waves per workgroup;
//   * larger M: smaller lane groups and more rows per group, so that each
//     activation load feeds more weight rows, with fewer steps in flight to
//     bound register pressure.
#include <algorithm>

#include "gemv_kernels.hpp"
#include "mfma_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

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

template <int M, int GS, int R, int U, int WPB>
hipError_t run_fp8(const F8Args& a, hipStream_t st) {
    constexpr int rows_per_block = (64 / GS) * R * WPB;
    dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((gemv_fp8_kernel<M, GS, R, U, WPB>), grid, dim3(64 * WPB), 0, st,
                       a.x, a.ldx, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
    return hipGetLastError();
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


// Matrix-core kernels: one workgroup of kMfmaKS waves per 16-row tile, U
// chunks of 256 K per batch (U = the chunks of a wave's K slice, at most 5).
inline int mfma_u(int64_t K) {
    const int64_t nch = (K + 255) >> 8, per = (nch + kMfmaKS - 1) / kMfmaKS;
    return (int)(per < 5 ? (per < 1 ? 1 : per) : 5);
}

#define QLIN_BY_U(KERNEL, U_, ...)                                                        \
    switch (U_) {                                                                        \
        case 1: hipLaunchKernelGGL((KERNEL<1>), __VA_ARGS__); break;                     \
        case 2: hipLaunchKernelGGL((KERNEL<2>), __VA_ARGS__); break;                     \
        case 3: hipLaunchKernelGGL((KERNEL<3>), __VA_ARGS__); break;                     \
        case 4: hipLaunchKernelGGL((KERNEL<4>), __VA_ARGS__); break;                     \
        default: hipLaunchKernelGGL((KERNEL<5>), __VA_ARGS__); break;                    \
    }

hipError_t run_i8_mfma(const I8Args& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * kMfmaKS);
    QLIN_BY_U(gemv_i8_mfma_kernel, mfma_u(a.K), grid, block, 0, st, a.xq, a.ldxq, a.xs, a.xs_step, (int)a.M,
              a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.bias, a.y, a.ldy, a.out_kind)
    return hipGetLastError();
}

hipError_t run_fp8_mfma(const F8Args& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * kMfmaKS);
    QLIN_BY_U(gemv_fp8_mfma_kernel, mfma_u(a.K), grid, block, 0, st, a.x, a.ldx, (int)a.M, a.K, a.w, a.ldw,
              a.N, a.ws, a.ws_step, a.y, a.ldy)
    return hipGetLastError();
}

hipError_t run_blk_mfma(const BlkArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * kMfmaKS);
    QLIN_BY_U(gemv_fp8_blk_mfma_kernel, mfma_u(a.K), grid, block, 0, st, a.xq, a.xs, (int)a.M, a.K, a.w,
              a.ldw, a.N, a.ws, a.y, a.ldy)
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_i8(const I8Args& a, hipStream_t st) {
    switch (a.M) {
        case 1: QLIN_M1_BY_STEPS(run_i8, a, st)
        case 2: return run_i8<2, 32, 2, 2, 1>(a, st);
        case 3: return run_i8<3, 32, 4, 1, 1>(a, st);
        default: return run_i8_mfma(a, st);
    }
}

hipError_t launch_gemv_fp8(const F8Args& a, hipStream_t st) {
    switch (a.M) {
        case 1: return run_fp8<1, 32, 2, 1, 1>(a, st);
        case 2: return run_fp8<2, 64, 4, 1, 1>(a, st);
        case 3: return run_fp8<3, 64, 4, 1, 1>(a, st);
        default: return run_fp8_mfma(a, st);
    }
}

hipError_t launch_gemv_fp8_blk(const BlkArgs& a, hipStream_t st) {
    switch (a.M) {
        case 1: return run_blk<1, 64, 1, 2, 4>(a, st);
        default: return run_blk_mfma(a, st);
    }
}

}  // namespace qlin
