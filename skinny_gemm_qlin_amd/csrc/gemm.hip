// gemm.hip -- launchers of the prefill GEMM (gemm_kernels.hpp), used by the
// dense entry points when M > 16.
#include "gemm_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

namespace {

template <int WF, int ACT, int EPI, int TN = 4, int TM = 4, int BK = 64>
hipError_t run_gemm(const GemmParams& p, hipStream_t st) {
    constexpr int BN = GemmShape<TN, TM, BK>::BN, BM = GemmShape<TN, TM, BK>::BM;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const int64_t grid = (tiles + 7) / 8 * 8;  // the XCD remap needs a multiple of 8
    hipLaunchKernelGGL((gemm_kernel<WF, ACT, EPI, TN, TM, BK>), dim3((unsigned)grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int WF, int ACT, int EPI, int BN, int BM, int NW = 4>
hipError_t run_gemm_dma(const GemmParams& p, hipStream_t st) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const int64_t grid = (tiles + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_dma_kernel<WF, ACT, EPI, BN, BM, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st, p);
    return hipGetLastError();
}

// Direct-to-LDS kernel, one-byte operands, K % 128 == 0.  Tiles (weight rows
// x tokens, measured with INT8 at N = 17408, K = 5120): 64 x 64 up to 256
// tokens, 64 x 128 up to 1024 and 128 x 128 above, both with 8 waves.
template <int WF, int ACT, int EPI>
hipError_t run_dma(const GemmParams& p, hipStream_t st) {
    if (p.M <= 256) return run_gemm_dma<WF, ACT, EPI, 64, 64>(p, st);
    if (p.M <= 1024) return run_gemm_dma<WF, ACT, EPI, 64, 128, 8>(p, st);
    return run_gemm_dma<WF, ACT, EPI, 128, 128, 8>(p, st);
}

}  // namespace

// Tile choice (measured at N = 17408, K = 5120): up to 256 tokens the 64 x 64
// tiles give 4x more workgroups (the GEMM is latency-bound there); above,
// 128 x 128 tiles.  INT8 takes K tiles of 128 (one 64-deep MFMA step per
// 64 bytes would double the barriers per MFMA).
constexpr int64_t kSmallTileMaxM = 256;

hipError_t launch_gemm_i8(const I8Args& a, hipStream_t st) {
    GemmParams p{a.xq, a.ldxq, a.xs, a.xs_step, nullptr, a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step,
                 nullptr, a.bias, a.y, a.ldy, a.out_kind};
    if (a.K % 128 == 0) return run_dma<kFmtE4M3, kActI8, kEpiI8>(p, st);
    if (a.M <= kSmallTileMaxM) return run_gemm<kFmtE4M3, kActI8, kEpiI8, 2, 2, 128>(p, st);
    return run_gemm<kFmtE4M3, kActI8, kEpiI8, 4, 4, 128>(p, st);
}

hipError_t launch_gemm_fp8(const F8Args& a, hipStream_t st) {
    GemmParams p{a.x, a.ldx, nullptr, 0, nullptr, a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step,
                 nullptr, nullptr, a.y, a.ldy, 0};
    if (a.K % 128 == 0) {
        // bf16 activation rows are twice as wide, so the token side of the
        // tile stays at 64; above 256 tokens 8 waves of 32 x 32 share a
        // 128 x 64 tile (measured: M = 128 / 512 / 2048 / 4096 63.9 / 157.5 /
        // 572 / 1084 us; 4 waves on 128 x 64: 172 / 612 / 1121 us at the
        // larger M; the register-staged kernel 80 / 219 / 645 / 1220 us)
        if (a.M <= kSmallTileMaxM) return run_gemm_dma<kFmtE4M3, kActBf16, kEpiWs, 64, 64>(p, st);
        return run_gemm_dma<kFmtE4M3, kActBf16, kEpiWs, 128, 64, 8>(p, st);
    }
    if (a.M <= kSmallTileMaxM) return run_gemm<kFmtE4M3, kActBf16, kEpiWs, 2, 2, 64>(p, st);
    return run_gemm<kFmtE4M3, kActBf16, kEpiWs, 4, 4, 64>(p, st);
}

hipError_t launch_gemm_fp8_w8a8(const W8A8F8Args& a, hipStream_t st) {
    GemmParams p{a.xq, a.ldxq, a.xs, a.xs_step, nullptr, a.M, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step,
                 nullptr, nullptr, a.y, a.ldy, 0};
    if (a.K % 128 == 0) {
        if (a.x_fmt == kFmtE5M2)
            return a.w_fmt == kFmtE5M2 ? run_dma<kFmtE5M2, kActE5M2, kEpiXsWs>(p, st)
                                       : run_dma<kFmtE4M3, kActE5M2, kEpiXsWs>(p, st);
        return a.w_fmt == kFmtE5M2 ? run_dma<kFmtE5M2, kActE4M3, kEpiXsWs>(p, st)
                                   : run_dma<kFmtE4M3, kActE4M3, kEpiXsWs>(p, st);
    }
    const bool small = a.M <= kSmallTileMaxM;
    if (a.x_fmt == kFmtE5M2) {
        if (a.w_fmt == kFmtE5M2)
            return small ? run_gemm<kFmtE5M2, kActE5M2, kEpiXsWs, 2, 2, 64>(p, st)
                         : run_gemm<kFmtE5M2, kActE5M2, kEpiXsWs, 4, 4, 128>(p, st);
        return small ? run_gemm<kFmtE4M3, kActE5M2, kEpiXsWs, 2, 2, 64>(p, st)
                     : run_gemm<kFmtE4M3, kActE5M2, kEpiXsWs, 4, 4, 128>(p, st);
    }
    if (a.w_fmt == kFmtE5M2)
        return small ? run_gemm<kFmtE5M2, kActE4M3, kEpiXsWs, 2, 2, 64>(p, st)
                     : run_gemm<kFmtE5M2, kActE4M3, kEpiXsWs, 4, 4, 128>(p, st);
    return small ? run_gemm<kFmtE4M3, kActE4M3, kEpiXsWs, 2, 2, 64>(p, st)
                 : run_gemm<kFmtE4M3, kActE4M3, kEpiXsWs, 4, 4, 128>(p, st);
}

// Block FP8 at any block shape (block_k a multiple of 32; K % 128 == 0).
hipError_t launch_gemm_fp8_blkg(const BlkArgs& a, int64_t bn, int64_t bk, hipStream_t st) {
    GemmParams p{a.xq, a.K, nullptr, 0, a.xs, a.M, a.K, a.w, a.ldw, a.N, nullptr, 0,
                 a.ws, nullptr, a.y, a.ldy, 0, bn, bk};
    const bool word = (((uintptr_t)a.ws | (uintptr_t)a.xs) & 3) == 0, half = (((uintptr_t)a.ws | (uintptr_t)a.xs) & 1) == 0;
    if (bk == 32 && word) return run_dma<kFmtE4M3, kActE4M3, kEpiBlkGW>(p, st);
    if (bk == 64 && half) return run_dma<kFmtE4M3, kActE4M3, kEpiBlkGH>(p, st);
    if (bk % 128 == 0) return run_dma<kFmtE4M3, kActE4M3, kEpiBlkGT>(p, st);
    return run_dma<kFmtE4M3, kActE4M3, kEpiBlkG>(p, st);
}

hipError_t launch_gemm_fp8_blk(const BlkArgs& a, hipStream_t st) {
    GemmParams p{a.xq, a.K, nullptr, 0, a.xs, a.M, a.K, a.w, a.ldw, a.N, nullptr, 0,
                 a.ws, nullptr, a.y, a.ldy, 0};
    return run_dma<kFmtE4M3, kActE4M3, kEpiBlk>(p, st);  // K % 128 == 0 by contract
}

}  // namespace qlin
