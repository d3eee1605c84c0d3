// gemv.hip -- skinny GEMV kernels for gfx950 (VALU path, M = 1..16).
//
// Work split (same for the three weight formats):
//   * one wavefront per workgroup; the wave is 4 DPP rows ("groups") of 16
//     lanes, and group g owns R consecutive weight rows;
//   * a group walks K in steps of 16 chunks; lane j of the group reads chunk
//     c = 16*step + j, i.e. 16 bytes of each of its R rows with one 128-bit
//     load, so a group reads 256 contiguous bytes of a row per step (two
//     whole 128-byte lines) and every weight byte is loaded exactly once;
//   * the matching x chunk is loaded once per step and reused for the R rows;
//   * after the K loop each lane holds R*M partial sums; a DPP row_ror tree
//     (4 adds) reduces them over the 16 lanes of the group, and the epilogue
//     for value v runs in lane v % 16.
// No atomics, no cross-workgroup reduction: results are deterministic.
#include "qlin_device.hpp"
#include "qlin_launch.hpp"

namespace qlin {

// ------------------------------------------------------------------ INT8
// acc = sum_k xq*w with v_dot4 (exact int32); epilogue bf16((acc*xs)*ws)
// [Z100 operator-family table, INT8 row; section 2.1].
template <int M, int R, int U>
__global__ __launch_bounds__(64) void gemv_i8_kernel(
    const int8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step,
    int64_t K, const int8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int out_kind) {
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + g) * R;
    const int8_t* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w + (n0 + r < N ? n0 + r : N - 1) * ldw;

    int acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0;

    const int64_t nchunk = K >> 4;          // 16 int8 per chunk
    const int64_t full = nchunk >> 4;       // steps where all 16 lanes have a chunk
    int64_t s = 0;
    for (; s + U <= full; s += U) {
        u32x4_t wv[U][R], xv[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r) wv[u][r] = ld_stream(wr[r] + ((s + u) * 16 + j) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m) xv[u][m] = ld16(xq + m * ldxq + ((s + u) * 16 + j) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    int a = acc[r][m];
                    a = sdot4(wv[u][r].x, xv[u][m].x, a);
                    a = sdot4(wv[u][r].y, xv[u][m].y, a);
                    a = sdot4(wv[u][r].z, xv[u][m].z, a);
                    a = sdot4(wv[u][r].w, xv[u][m].w, a);
                    acc[r][m] = a;
                }
    }
    for (; s * 16 < nchunk; ++s) {
        const int64_t c = s * 16 + j;
        if (c < nchunk) {
            u32x4_t wv[R], xv[M];
#pragma unroll
            for (int r = 0; r < R; ++r) wv[r] = ld_stream(wr[r] + c * 16);
#pragma unroll
            for (int m = 0; m < M; ++m) xv[m] = ld16(xq + m * ldxq + c * 16);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    int a = acc[r][m];
                    a = sdot4(wv[r].x, xv[m].x, a);
                    a = sdot4(wv[r].y, xv[m].y, a);
                    a = sdot4(wv[r].z, xv[m].z, a);
                    a = sdot4(wv[r].w, xv[m].w, a);
                    acc[r][m] = a;
                }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = row_sum_i32(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v & 15) == j && n < N) {
                if (out_kind == 1) {
                    ((int32_t*)y)[m * ldy + n] = acc[r][m];
                } else {
                    float t = (float)acc[r][m];
                    t = t * xs[m * xs_step];
                    t = t * ws[n * ws_step];
                    uint16_t o = f32_to_bf16(t);
                    if (bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(bias[n]));
                    ((uint16_t*)y)[m * ldy + n] = o;
                }
            }
        }
}

// ------------------------------------------------------------------ FP8 weight-only
// y = bf16(ws[n] * sum_k e4m3(w)*x): E4M3 -> bf16 by the hardware convert,
// v_dot2_f32_bf16 with fp32 accumulation, the scale multiplied once
// [Z100 operator-family table, FP8 row; section 2.2].
__device__ __forceinline__ void fp8_chunk_dot(const u32x4_t& wv, const u32x4_t& xa, const u32x4_t& xb,
                                              float& acc, const bf16x2_t wb[8]) {
    float a = acc;
    a = dot2(wb[0], as_bf16x2(xa.x), a);
    a = dot2(wb[1], as_bf16x2(xa.y), a);
    a = dot2(wb[2], as_bf16x2(xa.z), a);
    a = dot2(wb[3], as_bf16x2(xa.w), a);
    a = dot2(wb[4], as_bf16x2(xb.x), a);
    a = dot2(wb[5], as_bf16x2(xb.y), a);
    a = dot2(wb[6], as_bf16x2(xb.z), a);
    a = dot2(wb[7], as_bf16x2(xb.w), a);
    acc = a;
}

__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4_t& wv, bf16x2_t wb[8]) {
    e4m3x4_to_bf16(wv.x, wb[0], wb[1]);
    e4m3x4_to_bf16(wv.y, wb[2], wb[3]);
    e4m3x4_to_bf16(wv.z, wb[4], wb[5]);
    e4m3x4_to_bf16(wv.w, wb[6], wb[7]);
}

template <int M, int R, int U>
__global__ __launch_bounds__(64) void gemv_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y, int64_t ldy) {
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + g) * R;
    const uint8_t* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w + (n0 + r < N ? n0 + r : N - 1) * ldw;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    const int64_t nchunk = K >> 4;  // 16 codes per chunk
    const int64_t full = nchunk >> 4;
    int64_t s = 0;
    for (; s + U <= full; s += U) {
        u32x4_t wv[U][R], xa[U][M], xb[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r) wv[u][r] = ld_stream(wr[r] + ((s + u) * 16 + j) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint16_t* xp = x + m * ldx + ((s + u) * 16 + j) * 16;
                xa[u][m] = ld16(xp);
                xb[u][m] = ld16(xp + 8);
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                bf16x2_t wb[8];
                e4m3x16_to_bf16(wv[u][r], wb);
#pragma unroll
                for (int m = 0; m < M; ++m) fp8_chunk_dot(wv[u][r], xa[u][m], xb[u][m], acc[r][m], wb);
            }
    }
    for (; s * 16 < nchunk; ++s) {
        const int64_t c = s * 16 + j;
        if (c < nchunk) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                u32x4_t wv = ld_stream(wr[r] + c * 16);
                bf16x2_t wb[8];
                e4m3x16_to_bf16(wv, wb);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint16_t* xp = x + m * ldx + c * 16;
                    fp8_chunk_dot(wv, ld16(xp), ld16(xp + 8), acc[r][m], wb);
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = row_sum_f32(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v & 15) == j && n < N) y[m * ldy + n] = f32_to_bf16(acc[r][m] * ws[n * ws_step]);
        }
}

// ------------------------------------------------------------------ block-scaled FP8
// out = sum_kb (sum_{k in kb} xq*w) * 2^(xs-127) * 2^(ws-127); each chunk of
// 16 codes lies inside one 128-wide block, so a lane folds the block scales
// into its own chunk partial before any reduction
// [Z100 section 2.4, block formula and scale-folding identity].
template <int M, int R, int U>
__global__ __launch_bounds__(64) void gemv_fp8_blk_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const uint8_t* __restrict__ ws, uint16_t* __restrict__ y, int64_t ldy) {
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + g) * R;
    const int64_t nkb = K >> 7;
    const uint8_t* wr[R];
    const uint8_t* wsr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        wr[r] = w + n * ldw;
        wsr[r] = ws + (n >> 7) * nkb;
    }

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    const int64_t nchunk = K >> 4;  // K % 128 == 0, so every step is full (16 chunks = 2 blocks)
    for (int64_t s = 0; s * 16 < nchunk; s += U) {
        u32x4_t wv[U][R], xv[U][M];
        float sw[U][R], sx[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * 16 + j;
            const bool ok = c < nchunk;
            const int64_t cc = ok ? c : 0;
            const int64_t kb = cc >> 3;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                wv[u][r] = ok ? ld_stream(wr[r] + cc * 16) : u32x4_t{0, 0, 0, 0};
                sw[u][r] = ok ? ue8m0_to_f32(wsr[r][kb]) : 0.0f;  // idle lanes add exactly 0
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                xv[u][m] = ok ? ld16(xq + m * K + cc * 16) : u32x4_t{0, 0, 0, 0};
                sx[u][m] = ok ? ue8m0_to_f32(xs[m * nkb + kb]) : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bf16x2_t xb[M][8];
#pragma unroll
            for (int m = 0; m < M; ++m) e4m3x16_to_bf16(xv[u][m], xb[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                bf16x2_t wb[8];
                e4m3x16_to_bf16(wv[u][r], wb);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float loc = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) loc = dot2(wb[i], xb[m][i], loc);
                    acc[r][m] += (loc * sx[u][m]) * sw[u][r];
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = row_sum_f32(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v & 15) == j && n < N) y[m * ldy + n] = f32_to_bf16(acc[r][m]);
        }
}

// ------------------------------------------------------------------ launchers
// Tile shape per M: R rows per 16-lane group, U K-steps unrolled (loads in
// flight per lane = U*(R + M*xloads)).
template <int M> struct I8Tile { static constexpr int R = M <= 2 ? 1 : (M <= 8 ? 2 : 4); static constexpr int U = M <= 1 ? 8 : (M <= 2 ? 4 : (M <= 4 ? 2 : 1)); };
template <int M> struct F8Tile { static constexpr int R = M <= 2 ? 1 : 2; static constexpr int U = M <= 1 ? 4 : (M <= 2 ? 2 : 1); };
template <int M> struct BlkTile { static constexpr int R = M <= 4 ? 1 : 2; static constexpr int U = M <= 2 ? 2 : 1; };

template <int M>
static hipError_t launch_i8_m(const I8Args& a, hipStream_t st) {
    constexpr int R = I8Tile<M>::R, U = I8Tile<M>::U;
    dim3 grid((unsigned)((a.N + 4 * R - 1) / (4 * R)));
    hipLaunchKernelGGL((gemv_i8_kernel<M, R, U>), grid, dim3(64), 0, st,
                       a.xq, a.ldxq, a.xs, a.xs_step, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step,
                       a.bias, a.y, a.ldy, a.out_kind);
    return hipGetLastError();
}

template <int M>
static hipError_t launch_fp8_m(const F8Args& a, hipStream_t st) {
    constexpr int R = F8Tile<M>::R, U = F8Tile<M>::U;
    dim3 grid((unsigned)((a.N + 4 * R - 1) / (4 * R)));
    hipLaunchKernelGGL((gemv_fp8_kernel<M, R, U>), grid, dim3(64), 0, st,
                       a.x, a.ldx, a.K, a.w, a.ldw, a.N, a.ws, a.ws_step, a.y, a.ldy);
    return hipGetLastError();
}

template <int M>
static hipError_t launch_blk_m(const BlkArgs& a, hipStream_t st) {
    constexpr int R = BlkTile<M>::R, U = BlkTile<M>::U;
    dim3 grid((unsigned)((a.N + 4 * R - 1) / (4 * R)));
    hipLaunchKernelGGL((gemv_fp8_blk_kernel<M, R, U>), grid, dim3(64), 0, st,
                       a.xq, a.xs, a.K, a.w, a.ldw, a.N, a.ws, a.y, a.ldy);
    return hipGetLastError();
}

#define QLIN_DISPATCH_M(FN, M, ...)                                             \
    switch (M) {                                                                \
        case 1: return FN<1>(__VA_ARGS__);   case 2: return FN<2>(__VA_ARGS__);   \
        case 3: return FN<3>(__VA_ARGS__);   case 4: return FN<4>(__VA_ARGS__);   \
        case 5: return FN<5>(__VA_ARGS__);   case 6: return FN<6>(__VA_ARGS__);   \
        case 7: return FN<7>(__VA_ARGS__);   case 8: return FN<8>(__VA_ARGS__);   \
        case 9: return FN<9>(__VA_ARGS__);   case 10: return FN<10>(__VA_ARGS__); \
        case 11: return FN<11>(__VA_ARGS__); case 12: return FN<12>(__VA_ARGS__); \
        case 13: return FN<13>(__VA_ARGS__); case 14: return FN<14>(__VA_ARGS__); \
        case 15: return FN<15>(__VA_ARGS__); case 16: return FN<16>(__VA_ARGS__); \
        default: return hipErrorInvalidValue;                                   \
    }

hipError_t launch_gemv_i8(const I8Args& a, hipStream_t st) { QLIN_DISPATCH_M(launch_i8_m, a.M, a, st) }
hipError_t launch_gemv_fp8(const F8Args& a, hipStream_t st) { QLIN_DISPATCH_M(launch_fp8_m, a.M, a, st) }
hipError_t launch_gemv_fp8_blk(const BlkArgs& a, hipStream_t st) { QLIN_DISPATCH_M(launch_blk_m, a.M, a, st) }

}  // namespace qlin
