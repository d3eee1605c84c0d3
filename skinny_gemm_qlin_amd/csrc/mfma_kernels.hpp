// mfma_kernels.hpp -- matrix-core (MFMA) skinny-GEMV kernels for gfx950, used
// where the VALU kernels are issue-bound (larger M).
//
// Layout facts (checked on the hardware): for the 16x16 MFMAs the A operand
// of lane l holds row l%16, the B operand holds column l%16, the K slots of A
// and B pair up lane group by lane group (l/16), and D[row][col] lives in
// lane col + 16*(row/4), register row%4.  Because the K-slot order is free
// as long as A and B agree, each MFMA reads 16 contiguous bytes per lane.
//
// Work split: a workgroup of KS wavefronts owns a tile of 16 weight rows and
// splits K between its waves.  A wave reads its slice of the 16 rows with
// the fast row-contiguous pattern (one load instruction = 4 rows x 256
// bytes), writes each 16-byte piece to a small padded LDS tile and reads it
// back in MFMA A layout (a transpose through LDS), while the activation B
// operand is read straight from x.  After the K loop the KS 16x16 partial
// tiles are summed through LDS in a fixed order (deterministic) and wave 0
// runs the epilogue.  No atomics.
#pragma once
#include "qlin_device.hpp"

namespace qlin {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kTilePitch = 256 + 16;  // LDS row pitch of the transpose tile (bytes); the pad spreads banks
constexpr int kMfmaKS = 4;            // default waves per workgroup (K split)

// Load the 16 rows x 256 bytes of chunk c into registers (4 instructions,
// each 4 rows x 256 contiguous bytes).  Past the end of K the address is
// clamped inside the row (a cached duplicate) -- callers zero the matching
// activation, so it adds nothing.
struct TileLoader {
    const uint8_t* row[4];
    int lp;
    __device__ TileLoader(const uint8_t* w, int64_t ldw, int64_t n0, int64_t N) {
        const int lane = threadIdx.x & 63;
        const int lr = lane >> 4;
        lp = lane & 15;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + 4 * q + lr;
            row[q] = w + (n < N ? n : N - 1) * ldw;
        }
    }
    __device__ __forceinline__ void load(u32x4_t v[4], int64_t c, int64_t K) const {
        const int64_t k = c * 256 + lp * 16;
        const int64_t kc = k < K ? k : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld_stream(row[q] + kc);
    }
};

// Write 4 loaded pieces into the wave's LDS tile (row 4q + lane/16, column
// 16*(lane%16)), i.e. the tile holds 16 rows x 256 bytes.
__device__ __forceinline__ void tile_store(uint8_t* t, const u32x4_t v[4]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane >> 4, lp = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4_t*)(t + (4 * q + lr) * kTilePitch + lp * 16) = v[q];
}

// 16 bytes of row lane%16 at byte offset off + 16*(lane/16) of the tile.
__device__ __forceinline__ u32x4_t tile_read(const uint8_t* t, int off) {
    const int lane = threadIdx.x & 63;
    return *(const u32x4_t*)(t + (lane & 15) * kTilePitch + off + 16 * (lane >> 4));
}

// Sum the KS partial accumulator tiles of the workgroup in wave order; returns
// true in wave 0, which then holds the total.
template <int KS, class T>
__device__ __forceinline__ bool ks_reduce(T& acc, T (*red)[64]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    red[wv][lane] = acc;
    __syncthreads();
    if (wv != 0) return false;
#pragma unroll
    for (int q = 1; q < KS; ++q) acc += red[q][lane];
    return true;
}

// 8 E4M3 codes (one uint2) -> one bf16x8 MFMA operand, exact.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8_e4m3(uint2 c) {
    bf16x2_t b[4];
    e4m3x4_to_bf16(c.x, b[0], b[1]);
    e4m3x4_to_bf16(c.y, b[2], b[3]);
    return bf16x8_t{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
}

// 16 E4M3 codes -> two bf16x8 MFMA operands (bytes 0-7, bytes 8-15), exact.
__device__ __forceinline__ void e4m3x16_to_bf16x8x2(const u32x4_t& c, bf16x8_t& lo, bf16x8_t& hi) {
    bf16x2_t b[8];
    e4m3x4_to_bf16(c.x, b[0], b[1]);
    e4m3x4_to_bf16(c.y, b[2], b[3]);
    e4m3x4_to_bf16(c.z, b[4], b[5]);
    e4m3x4_to_bf16(c.w, b[6], b[7]);
    lo = bf16x8_t{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
    hi = bf16x8_t{b[4][0], b[4][1], b[5][0], b[5][1], b[6][0], b[6][1], b[7][0], b[7][1]};
}

// Token block of a workgroup: blockIdx.y selects 16 tokens.  At decode the
// grid has one block row (blockIdx.y = 0, M <= 16); a prefill-sized call on
// a matrix too small to fill the chip runs these kernels over a grid of
// token blocks, so that each 16-row tile's K is still split between KS waves
// (split-K inside the workgroup, reduced in wave order: deterministic).
__device__ __forceinline__ int token_block_start() { return (int)blockIdx.y * 16; }
__device__ __forceinline__ int token_block_size(int M) {
    const int r = M - token_block_start();
    return r < 16 ? r : 16;
}

// ------------------------------------------------------------------ INT8 W8A8 (v_mfma_i32_16x16x64_i8)
// acc exact in int32; epilogue bf16((acc*xs)*ws) (+ bias) as the VALU kernel
// [Z100 operator-family table, INT8 row; section 2.1].
template <int U, int KS = kMfmaKS>
__global__ __launch_bounds__(64 * KS) void gemv_i8_mfma_kernel(
    const int8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step, int M,
    int64_t K, const int8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int out_kind) {
    {
        const int mb = token_block_start();
        xq += mb * ldxq;
        if (xs) xs += mb * xs_step;  // out_kind 1 may pass no scales
        y = (uint8_t*)y + mb * ldy * (out_kind == 1 ? 4 : 2);
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][16 * kTilePitch];
    __shared__ i32x4_t red[KS][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const TileLoader tl((const uint8_t*)w, ldw, n0, N);
    const bool xon = mi < M;
    const int8_t* xr = xq + (xon ? mi : 0) * ldxq;
    uint8_t* t = tile[wv];

    i32x4_t acc = {0, 0, 0, 0};
    for (int64_t c = c0; c < c1; c += U) {
        u32x4_t wv_[U][4], xb[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) tl.load(wv_[u], c + u < c1 ? c + u : c1 - 1, K);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int64_t k = (c + u) * 256 + 64 * h + 16 * mg;
                const bool ok = (c + u < c1) && k < K && xon;
                const u32x4_t v = ld16(xr + (ok ? k : 0));
                xb[u][h] = ok ? v : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tile_store(t, wv_[u]);
#pragma unroll
            for (int h = 0; h < 4; ++h)
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, tile_read(t, 64 * h)),
                                                           __builtin_bit_cast(i32x4_t, xb[u][h]), acc, 0, 0, 0);
        }
    }
    if (!ks_reduce<KS>(acc, red)) return;
    if (mi < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * mg + r;
            if (n >= N) continue;
            if (out_kind == 1) {
                ((int32_t*)y)[mi * ldy + n] = acc[r];
            } else {
                float v = (float)acc[r];
                v = v * xs[mi * xs_step];
                v = v * ws[n * ws_step];
                uint16_t o = f32_to_bf16(v);
                if (bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(bias[n]));
                ((uint16_t*)y)[mi * ldy + n] = o;
            }
        }
    }
}

// Activation rows staged like the weights: 16 token rows x 256 bytes per
// chunk, loaded 4 rows x 256 contiguous bytes per instruction (rows past M
// repeat row M-1: their output columns are not stored; bytes past K are 0).
struct XTileLoader {
    const uint8_t* row[4];
    int lp;
    __device__ XTileLoader(const uint8_t* x, int64_t ldx, int M) {
        const int lane = threadIdx.x & 63;
        const int lr = lane >> 4;
        lp = lane & 15;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * q + lr;
            row[q] = x + (int64_t)(m < M ? m : M - 1) * ldx;
        }
    }
    __device__ __forceinline__ void load(u32x4_t v[4], int64_t c, int64_t K, bool live) const {
        const int64_t k = c * 256 + lp * 16;
        const bool ok = live && k < K;
        const int64_t kc = ok ? k : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4_t t = ld16(row[q] + kc);
            v[q] = ok ? t : u32x4_t{0, 0, 0, 0};
        }
    }
};

// INT8 with the activation operand staged through a second per-wave LDS tile
// (row-contiguous loads instead of a 16-token gather per MFMA), shared by
// RT row tiles of 16 weight rows per wave.
template <int U, int KS = kMfmaKS, int RT = 1>
__global__ __launch_bounds__(64 * KS) void gemv_i8_mfma_xl_kernel(
    const int8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step, int M,
    int64_t K, const int8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int out_kind) {
    {
        const int mb = token_block_start();
        xq += mb * ldxq;
        if (xs) xs += mb * xs_step;  // out_kind 1 may pass no scales
        y = (uint8_t*)y + mb * ldy * (out_kind == 1 ? 4 : 2);
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][RT][16 * kTilePitch];
    __shared__ __align__(16) uint8_t xtile[KS][16 * kTilePitch];
    __shared__ i32x4_t red[KS][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t nb = (int64_t)blockIdx.x * 16 * RT;
    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const XTileLoader xl((const uint8_t*)xq, ldxq, M);
    uint8_t* xt = xtile[wv];

    i32x4_t acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r] = i32x4_t{0, 0, 0, 0};
    for (int64_t c = c0; c < c1; c += U) {
        u32x4_t wv_[U][RT][4], xv_[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const TileLoader tl((const uint8_t*)w, ldw, nb + 16 * r, N);
                tl.load(wv_[u][r], c + u < c1 ? c + u : c1 - 1, K);
            }
#pragma unroll
        for (int u = 0; u < U; ++u) xl.load(xv_[u], c + u, K, c + u < c1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tile_store(xt, xv_[u]);
#pragma unroll
            for (int r = 0; r < RT; ++r) tile_store(tile[wv][r], wv_[u][r]);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const i32x4_t bx = __builtin_bit_cast(i32x4_t, tile_read(xt, 64 * h));
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        __builtin_bit_cast(i32x4_t, tile_read(tile[wv][r], 64 * h)), bx, acc[r], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (rt) __syncthreads();  // wave 0 is done reading red
        if (!ks_reduce<KS>(acc[rt], red)) continue;
        if (mi < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = nb + 16 * rt + 4 * mg + r;
                if (n >= N) continue;
                if (out_kind == 1) {
                    ((int32_t*)y)[mi * ldy + n] = acc[rt][r];
                } else {
                    float v = (float)acc[rt][r];
                    v = v * xs[mi * xs_step];
                    v = v * ws[n * ws_step];
                    uint16_t o = f32_to_bf16(v);
                    if (bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(bias[n]));
                    ((uint16_t*)y)[mi * ldy + n] = o;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ FP8-E4M3 weight-only (v_mfma_f32_16x16x32_bf16)
// The E4M3 codes read back from the tile are converted to bf16 (exact) and
// multiplied with the bf16 activations; fp32 accumulation; the weight scale
// once in the epilogue [Z100 operator-family table, FP8 row; section 2.2].
// MFMA (h, half) of a chunk covers K = c*256 + 64h + 16g + 8*half + [0, 8).
template <int U, int KS = kMfmaKS>
__global__ __launch_bounds__(64 * KS) void gemv_fp8_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y, int64_t ldy) {
    {
        const int mb = token_block_start();
        x += mb * ldx;
        y += mb * ldy;
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][16 * kTilePitch];
    __shared__ f32x4_t red[KS][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const TileLoader tl(w, ldw, n0, N);
    const bool xon = mi < M;
    const uint16_t* xr = x + (xon ? mi : 0) * ldx;
    uint8_t* t = tile[wv];

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t c = c0; c < c1; c += U) {
        u32x4_t wv_[U][4], xb[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) tl.load(wv_[u], c + u < c1 ? c + u : c1 - 1, K);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < 8; ++h) {  // h = 2*(64-K slice) + half
                const int64_t k = (c + u) * 256 + 64 * (h >> 1) + 16 * mg + 8 * (h & 1);
                const bool ok = (c + u < c1) && k < K && xon;
                const u32x4_t v = ld16(xr + (ok ? k : 0));
                xb[u][h] = ok ? v : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tile_store(t, wv_[u]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t a0, a1;
                e4m3x16_to_bf16x8x2(tile_read(t, 64 * s), a0, a1);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8_t, xb[u][2 * s]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, xb[u][2 * s + 1]), acc, 0, 0, 0);
            }
        }
    }
    if (!ks_reduce<KS>(acc, red)) return;
    if (mi < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * mg + r;
            if (n < N) y[mi * ldy + n] = f32_to_bf16(acc[r] * ws[n * ws_step]);
        }
    }
}

// ------------------------------------------------------------------ FP8 W8A8 (v_mfma_f32_16x16x32_bf16)
// Weight codes (format WF) from the tile and activation codes (format XF)
// straight from xq, each widened to bf16 (exact) for the bf16 matrix core
// with fp32 accumulation; epilogue bf16((acc*xs)*ws) as the VALU kernel
// [Z100 operator-family table, FP8 row (W8A8); section 2.2].
template <int F>
__device__ __forceinline__ void fp8x16_to_bf16x8x2(const u32x4_t& c, bf16x8_t& lo, bf16x8_t& hi) {
    bf16x2_t b[8];
    fp8x4_to_bf16<F>(c.x, b[0], b[1]);
    fp8x4_to_bf16<F>(c.y, b[2], b[3]);
    fp8x4_to_bf16<F>(c.z, b[4], b[5]);
    fp8x4_to_bf16<F>(c.w, b[6], b[7]);
    lo = bf16x8_t{b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
    hi = bf16x8_t{b[4][0], b[4][1], b[5][0], b[5][1], b[6][0], b[6][1], b[7][0], b[7][1]};
}

// XL: the activation codes are staged through a per-wave LDS tile like the
// weights (row-contiguous loads), for the larger token counts.
template <int U, int KS, int XF, int WF, bool XL = false>
__global__ __launch_bounds__(64 * KS) void gemv_fp8_w8a8_mfma_kernel(
    const uint8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step, int M,
    int64_t K, const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y, int64_t ldy) {
    {
        const int mb = token_block_start();
        xq += mb * ldxq;
        xs += mb * xs_step;
        y += mb * ldy;
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][16 * kTilePitch];
    __shared__ __align__(16) uint8_t xtile[XL ? KS : 1][16 * kTilePitch];
    __shared__ f32x4_t red[KS][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const TileLoader tl(w, ldw, n0, N);
    const bool xon = mi < M;
    const uint8_t* xr = xq + (xon ? mi : 0) * ldxq;
    uint8_t* t = tile[wv];

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const XTileLoader xtl(xq, ldxq, M);
    for (int64_t c = c0; c < c1; c += U) {
        u32x4_t wv_[U][4], xb[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) tl.load(wv_[u], c + u < c1 ? c + u : c1 - 1, K);
        if constexpr (XL) {
#pragma unroll
            for (int u = 0; u < U; ++u) xtl.load(xb[u], c + u, K, c + u < c1);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int64_t k = (c + u) * 256 + 64 * s4 + 16 * mg;
                    const bool ok = (c + u < c1) && k < K && xon;
                    const u32x4_t v = ld16(xr + (ok ? k : 0));
                    xb[u][s4] = ok ? v : u32x4_t{0, 0, 0, 0};
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tile_store(t, wv_[u]);
            if constexpr (XL) tile_store(xtile[wv], xb[u]);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                bf16x8_t a0, a1, b0, b1;
                fp8x16_to_bf16x8x2<WF>(tile_read(t, 64 * s4), a0, a1);
                fp8x16_to_bf16x8x2<XF>(XL ? tile_read(xtile[wv], 64 * s4) : xb[u][s4], b0, b1);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc, 0, 0, 0);
            }
        }
    }
    if (!ks_reduce<KS>(acc, red)) return;
    if (mi < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * mg + r;
            if (n < N) {
                float v = acc[r] * xs[mi * xs_step];
                v = v * ws[n * ws_step];
                y[mi * ldy + n] = f32_to_bf16(v);
            }
        }
    }
}

// ------------------------------------------------------------------ block-scaled FP8 (v_mfma_f32_16x16x32_bf16)
// Both operands are E4M3 codes (weights from the tile, activations from the
// block quantiser); each is widened to bf16 (exact) and multiplied on the
// bf16 matrix core, which accumulates in fp32.  (The fp8 matrix-core
// instruction was measured to sum its 128 products with only ~13 bits, so it
// is not used.)  The 4 MFMAs of one 128-wide K block accumulate into a block
// partial D, then the block scales are folded in before the running sum:
//   acc += (D * 2^(ws[n/128, kb]-127)) * 2^(xs[token, kb]-127)
// [Z100 section 2.4: block formula, fold per K block; DSV4 section 3.3].
// The 16 rows of a tile share one 128-row scale block (tiles are 16-aligned).
template <int U, int KS = kMfmaKS>
__global__ __launch_bounds__(64 * KS) void gemv_fp8_blk_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int M, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const uint8_t* __restrict__ ws, uint16_t* __restrict__ y, int64_t ldy) {
    {
        const int mb = token_block_start();
        xq += mb * K;
        xs += mb * (K >> 7);
        y += mb * ldy;
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][16 * kTilePitch];
    __shared__ f32x4_t red[KS][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nkb = K >> 7;
    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const TileLoader tl(w, ldw, n0, N);
    const bool xon = mi < M;
    const uint8_t* xr = xq + (xon ? mi : 0) * K;
    const uint8_t* xsr = xs + (xon ? mi : 0) * nkb;
    const uint8_t* wsr = ws + (n0 >> 7) * nkb;
    uint8_t* t = tile[wv];

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t c = c0; c < c1; c += U) {
        u32x4_t wv_[U][4], xb[U][4];
        float sw[U][2], sx[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) tl.load(wv_[u], c + u < c1 ? c + u : c1 - 1, K);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int64_t k = (c + u) * 256 + 64 * s4 + 16 * mg;
                const bool ok = (c + u < c1) && k < K && xon;
                const u32x4_t v = ld16(xr + (ok ? k : 0));
                xb[u][s4] = ok ? v : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t kb = (c + u) * 2 + b;
                const bool okb = (c + u < c1) && kb < nkb;
                const int64_t kbc = okb ? kb : 0;
                // An idle block (past the wave's range or past K) has zero
                // activation codes, so its partial D is a zero and folds in
                // as one whatever finite scales it meets: it reads block 0's
                // (a NaN weight scale there makes the tile's outputs NaN in
                // any case).  Selecting 0 for it instead (`okb ? scale : 0`)
                // had the compiler branch over each pair of byte loads and
                // wait for it on its own, a round trip per block (0.7 us of
                // a 10 us call at 4096 x 7168).
                sw[u][b] = ue8m0_to_f32(wsr[kbc]);
                sx[u][b] = ue8m0_to_f32(xsr[kbc]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tile_store(t, wv_[u]);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int s4 = 2 * b + s2;
                    bf16x8_t a0, a1, b0, b1;
                    e4m3x16_to_bf16x8x2(tile_read(t, 64 * s4), a0, a1);
                    e4m3x16_to_bf16x8x2(xb[u][s4], b0, b1);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, d, 0, 0, 0);
                }
                acc += (d * sx[u][b]) * sw[u][b];  // activation scale first, as every block kernel
            }
        }
    }
    if (!ks_reduce<KS>(acc, red)) return;
    if (mi < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * mg + r;
            if (n < N) y[mi * ldy + n] = f32_to_bf16(acc[r]);
        }
    }
}

// ------------------------------------------------------------------ block-scaled FP8, any block shape
// block_n x block_k weight blocks (block_k a multiple of 32, block_n >= 1,
// down to one scale per row) and block_k-wide activation groups.  Here the
// K slots of each MFMA are 32 contiguous K (lane group g takes 8g .. 8g+7),
// so one 16 x 16 x 32 MFMA lies inside one K block; its result accumulates
// in a block partial D that is folded when the block ends (or the wave's K
// range does): acc += (D * 2^(ws[row]-127)) * 2^(xs[token]-127), with a
// per-row weight scale (the 4 rows of a lane's D registers) and a per-token
// activation scale [Z100 section 2.4: block formula, fold per K block;
// block_n, block_k run-time parameters, block_k % 32].  The tile's scale
// bytes are staged once in LDS, transposed to [K block][16] so that a lane's
// 4 row scales are one 32-bit LDS word.
// PAIR (block_k a multiple of 64): the K slots of two MFMAs are paired over
// 64 K as in gemv_fp8_blk_mfma_kernel (16-byte loads of both operands per
// lane for two MFMAs); a 64-K step still lies in one block.
template <int KS, bool PAIR>
__global__ __launch_bounds__(64 * KS) void gemv_fp8_blkg_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int M, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const uint8_t* __restrict__ ws, int64_t bn, int64_t bk, uint16_t* __restrict__ y, int64_t ldy) {
    {
        const int mb = token_block_start();
        xq += mb * K;
        xs += mb * (K / bk);
        y += mb * ldy;
        M = token_block_size(M);
    }
    __shared__ __align__(16) uint8_t tile[KS][16 * kTilePitch];
    __shared__ f32x4_t red[KS][64];
    extern __shared__ __align__(16) uint8_t sct[];  // [nkb][16] weight scales, then [nkb][16] token scales
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nkb = K / bk;
    uint8_t* swt = sct;
    uint8_t* sxt = sct + nkb * 16;
    for (int64_t i = threadIdx.x; i < nkb * 16; i += 64 * KS) {
        const int r = (int)(i & 15);
        const int64_t kb = i >> 4;
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        swt[i] = ws[(n / bn) * nkb + kb];
        sxt[i] = r < M ? xs[r * nkb + kb] : (uint8_t)127;
    }
    __syncthreads();

    const int64_t nch = (K + 255) >> 8, per = (nch + KS - 1) / KS;
    const int64_t c0 = wv * per, c1 = c0 + per < nch ? c0 + per : nch;
    const TileLoader tl(w, ldw, n0, N);
    const uint8_t* xr = xq + (int64_t)(mi < M ? mi : M - 1) * K;
    uint8_t* t = tile[wv];

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
    int64_t kb_cur = -1, kb_end = 0;  // current K block and its end (K index)
    auto fold = [&]() {
        const uint32_t s4 = *(const uint32_t*)(swt + kb_cur * 16 + 4 * mg);
        const float sx = ue8m0_to_f32(sxt[kb_cur * 16 + mi]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += (d[r] * sx) * ue8m0_to_f32((s4 >> (8 * r)) & 0xFFu);
        d = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };
    constexpr int STEP = PAIR ? 64 : 32;
    for (int64_t c = c0; c < c1; ++c) {
        u32x4_t wv_[4];
        tl.load(wv_, c, K);
        tile_store(t, wv_);
#pragma unroll
        for (int j = 0; j < 256 / STEP; ++j) {
            const int64_t k0 = c * 256 + STEP * j;
            if (k0 >= K) break;  // wave-uniform; K % STEP == 0
            if (kb_cur < 0) {  // first step of this wave's K range
                kb_cur = k0 / bk;
                kb_end = (kb_cur + 1) * bk;
            } else if (k0 >= kb_end) {  // a step crosses at most one block boundary
                fold();
                ++kb_cur;
                kb_end += bk;
            }
            if constexpr (PAIR) {
                bf16x8_t a0, a1, b0, b1;
                e4m3x16_to_bf16x8x2(tile_read(t, 64 * j), a0, a1);
                e4m3x16_to_bf16x8x2(ld16(xr + k0 + 16 * mg), b0, b1);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, d, 0, 0, 0);
            } else {
                const bf16x8_t a = fp8x8_to_bf16x8_e4m3(*(const uint2*)(t + mi * kTilePitch + 32 * j + 8 * mg));
                const bf16x8_t b = fp8x8_to_bf16x8_e4m3(*(const uint2*)(xr + k0 + 8 * mg));
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d, 0, 0, 0);
            }
        }
    }
    if (kb_cur >= 0) fold();
    if (!ks_reduce<KS>(acc, red)) return;
    if (mi < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 4 * mg + r;
            if (n < N) y[mi * ldy + n] = f32_to_bf16(acc[r]);
        }
    }
}

}  // namespace qlin
