// gemv_kernels.hpp -- VALU skinny-GEMV kernel templates for gfx950.
//
// One template family serves the three dense weight formats.  Work split:
//   * a workgroup has WPB wavefronts; a wavefront is 64/GS lane groups of GS
//     lanes (GS = 16, 32 or 64) and each group owns R consecutive weight rows;
//   * a group walks K in steps of GS chunks of 16 bytes: lane j of the group
//     reads chunk c = GS*step + j of each of its rows with one 128-bit load, so
//     one load instruction covers 64/GS rows with GS*16 contiguous bytes each
//     (GS = 64: one whole 1 KB run of one row), every weight byte is read once;
//   * U steps are issued before any is consumed (U*R loads in flight per
//     lane); the ragged end of K is folded into the last batch by clamping
//     the chunk index inside the row (an L2 hit) and zeroing the activation;
//   * the activation chunk for a step is loaded once and reused for the R
//     rows; after the K loop each lane holds R*M partial sums, reduced over
//     the GS lanes of the group with DPP row_ror adds (and cross-row shuffles
//     for GS > 16); the epilogue of value v runs in lane v % GS.
// No atomics and no cross-workgroup reduction, so results are deterministic.
#pragma once
#include "qlin_device.hpp"

namespace qlin {

template <int GS>
__device__ __forceinline__ int group_sum(int v) {
    v = row_sum_i32(v);
    if (GS >= 32) v += __shfl_xor(v, 16);
    if (GS >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int GS>
__device__ __forceinline__ float group_sum(float v) {
    v = row_sum_f32(v);
    if (GS >= 32) v += __shfl_xor(v, 16);
    if (GS >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Row index owned by (group, r), clamped so that loads stay inside W.
template <int GS, int R, int WPB>
__device__ __forceinline__ int64_t first_row() {
    constexpr int GPW = 64 / GS;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    return (((int64_t)blockIdx.x * WPB + wv) * GPW + lane / GS) * R;
}

// 16 E4M3 codes -> 8 bf16 pairs (exact)
__device__ __forceinline__ void e4m3x16(const u32x4_t& v, bf16x2_t o[8]) {
    e4m3x4_to_bf16(v.x, o[0], o[1]);
    e4m3x4_to_bf16(v.y, o[2], o[3]);
    e4m3x4_to_bf16(v.z, o[4], o[5]);
    e4m3x4_to_bf16(v.w, o[6], o[7]);
}

// ------------------------------------------------------------------ INT8 W8A8
// acc = sum_k xq*w with v_dot4 (exact int32); epilogue bf16((acc*xs)*ws) then
// + bias [Z100 operator-family table, INT8 row; section 2.1].
template <int M, int GS, int R, int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_i8_kernel(
    const int8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step,
    int64_t K, const int8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int out_kind) {
    const int j = (threadIdx.x & 63) % GS;
    const int64_t n0 = first_row<GS, R, WPB>();
    const int8_t* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w + (n0 + r < N ? n0 + r : N - 1) * ldw;

    int acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0;

    const int64_t nchunk = K >> 4;  // 16 int8 per chunk
    const int64_t nsteps = (nchunk + GS - 1) / GS;
    for (int64_t s = 0; s < nsteps; s += U) {
        u32x4_t wv[U][R], xv[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * GS + j;
            const int64_t cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
            for (int r = 0; r < R; ++r) wv[u][r] = ld_stream(wr[r] + cc * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * GS + j;
            const int64_t cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4_t t = ld16(xq + m * ldxq + cc * 16);
                xv[u][m] = c < nchunk ? t : u32x4_t{0, 0, 0, 0};
            }
        }
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

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = group_sum<GS>(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v % GS) == j && n < N) {
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

// ------------------------------------------------------------------ FP8 W8A8
// Both operands are FP8 codes (activations XF, weights WF: E4M3 or E5M2),
// each widened to bf16 exactly by the hardware convert; a product of two
// such values is exact in fp32, so v_dot2 bf16 with fp32 accumulation only
// rounds the running sum.  Epilogue as the INT8 path: bf16((acc*xs)*ws)
// [Z100 operator-family table, FP8 row (W8A8); section 2.2].
template <int F>
__device__ __forceinline__ void fp8x16(const u32x4_t& v, bf16x2_t o[8]) {
    fp8x4_to_bf16<F>(v.x, o[0], o[1]);
    fp8x4_to_bf16<F>(v.y, o[2], o[3]);
    fp8x4_to_bf16<F>(v.z, o[4], o[5]);
    fp8x4_to_bf16<F>(v.w, o[6], o[7]);
}

template <int M, int GS, int R, int U, int WPB, int XF, int WF>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_w8a8_kernel(
    const uint8_t* __restrict__ xq, int64_t ldxq, const float* __restrict__ xs, int xs_step,
    int64_t K, const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y, int64_t ldy) {
    const int j = (threadIdx.x & 63) % GS;
    const int64_t n0 = first_row<GS, R, WPB>();
    const uint8_t* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w + (n0 + r < N ? n0 + r : N - 1) * ldw;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    const int64_t nchunk = K >> 4;  // 16 codes per chunk
    const int64_t nsteps = (nchunk + GS - 1) / GS;
    for (int64_t s = 0; s < nsteps; s += U) {
        u32x4_t wv[U][R], xv[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * GS + j;
            const int64_t cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
            for (int r = 0; r < R; ++r) wv[u][r] = ld_stream(wr[r] + cc * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * GS + j;
            const int64_t cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4_t t = ld16(xq + m * ldxq + cc * 16);
                xv[u][m] = c < nchunk ? t : u32x4_t{0, 0, 0, 0};  // code 0 decodes to +0 in both formats
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bf16x2_t xb[M][8];
#pragma unroll
            for (int m = 0; m < M; ++m) fp8x16<XF>(xv[u][m], xb[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                bf16x2_t wb[8];
                fp8x16<WF>(wv[u][r], wb);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float a = acc[r][m];
#pragma unroll
                    for (int i = 0; i < 8; ++i) a = dot2(wb[i], xb[m][i], a);
                    acc[r][m] = a;
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = group_sum<GS>(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v % GS) == j && n < N) {
                float t = acc[r][m] * xs[m * xs_step];
                t = t * ws[n * ws_step];
                y[m * ldy + n] = f32_to_bf16(t);
            }
        }
}

// ------------------------------------------------------------------ block-scaled FP8
// out = sum_kb (sum_{k in kb} xq*w) * 2^(xs-127) * 2^(ws-127).  A chunk of 16
// codes lies inside one 128-wide block (kb = c/8), so each lane multiplies the
// block scales into its own chunk partial before any reduction
// [Z100 section 2.4: block formula and scale-folding identity].
template <int M, int GS, int R, int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_blk_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const uint8_t* __restrict__ ws, uint16_t* __restrict__ y, int64_t ldy) {
    const int j = (threadIdx.x & 63) % GS;
    const int64_t n0 = first_row<GS, R, WPB>();
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

    const int64_t nchunk = K >> 4;
    const int64_t nsteps = (nchunk + GS - 1) / GS;
    for (int64_t s = 0; s < nsteps; s += U) {
        u32x4_t wv[U][R], xv[U][M];
        float sw[U][R], sx[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * GS + j;
            const bool ok = c < nchunk;
            const int64_t cc = ok ? c : nchunk - 1;
            const int64_t kb = cc >> 3;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                wv[u][r] = ld_stream(wr[r] + cc * 16);
                sw[u][r] = ok ? ue8m0_to_f32(wsr[r][kb]) : 0.0f;  // an idle lane adds exactly 0
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                xv[u][m] = ld16(xq + m * K + cc * 16);
                sx[u][m] = ok ? ue8m0_to_f32(xs[m * nkb + kb]) : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bf16x2_t xb[M][8];
#pragma unroll
            for (int m = 0; m < M; ++m) e4m3x16(xv[u][m], xb[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                bf16x2_t wb[8];
                e4m3x16(wv[u][r], wb);
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
        for (int m = 0; m < M; ++m) acc[r][m] = group_sum<GS>(acc[r][m]);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int v = r * M + m;
            const int64_t n = n0 + r;
            if ((v % GS) == j && n < N) y[m * ldy + n] = f32_to_bf16(acc[r][m]);
        }
}

// M = 1 block-scaled FP8 with the scale bytes fetched once per batch.  A wave
// owns one row; a step is 64 lanes x 16 bytes = 8 K blocks of 128.  For a
// batch of U <= 8 steps, lane l loads the weight and the activation scale of
// K block (first block of the batch) + l, and in step u the lanes read the
// scales of their own block (u*8 + lane/8) with a cross-lane shuffle instead
// of two more byte loads per step.  Arithmetic and order as
// gemv_fp8_blk_kernel: acc += (dot * 2^(xs-127)) * 2^(ws-127).
template <int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_blk_m1_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const uint8_t* __restrict__ ws, uint16_t* __restrict__ y) {
    static_assert(U >= 1 && U <= 8, "one scale byte per lane covers at most 8 steps");
    const int j = threadIdx.x & 63;
    const int64_t n = first_row<64, 1, WPB>();
    if (n >= N) return;  // wave-uniform
    const int64_t nkb = K >> 7;
    const uint8_t* wr = w + n * ldw;
    const uint8_t* wsr = ws + (n >> 7) * nkb;
    const int64_t nchunk = K >> 4;
    const int64_t nsteps = (nchunk + 63) >> 6;
    float acc = 0.0f;
    for (int64_t s = 0; s < nsteps; s += U) {
        const int64_t kbl = s * 8 + j;
        const bool okb = j < 8 * U && kbl < nkb;
        const float swl = okb ? ue8m0_to_f32(wsr[kbl]) : 0.0f;
        const float sxl = okb ? ue8m0_to_f32(xs[kbl]) : 0.0f;
        u32x4_t wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * 64 + j;
            const int64_t cc = c < nchunk ? c : nchunk - 1;
            wv[u] = ld_stream(wr + cc * 16);
            xv[u] = ld16(xq + cc * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = (s + u) * 64 + j < nchunk;
            const float sw = __shfl(swl, u * 8 + (j >> 3));
            const float sx = __shfl(sxl, u * 8 + (j >> 3));
            bf16x2_t xb[8], wb[8];
            e4m3x16(xv[u], xb);
            e4m3x16(wv[u], wb);
            float loc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) loc = dot2(wb[i], xb[i], loc);
            acc += ok ? (loc * sx) * sw : 0.0f;  // a lane past the row end adds 0
        }
    }
    acc = group_sum<64>(acc);
    if (j == 0) y[n] = f32_to_bf16(acc);
}

// M = 1 block-scaled FP8 with the activation quantisation fused in (one
// launch instead of two).  Each wave first issues the loads of its row's
// first batch of weights (after its first activation load), then the
// workgroup quantises the token's row into
// LDS (a 16-lane DPP row per 128-group, 8 values per lane, the rule of
// blk_act_quant_kernel: bit-identical codes) with the decoded group scales
// 2^(E-127), so the quantisation runs under the weights' HBM latency.  After
// one barrier each wave runs the gemv_fp8_blk_m1_kernel loop on its row with
// codes and scales read from LDS.  Group g is exported to xq / xs (each
// optional) by workgroup g % gridDim.x alone.  Dynamic LDS: K code bytes,
// then K/128 floats.
template <int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_blk_m1_fq_kernel(
    const uint16_t* __restrict__ x, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N, const uint8_t* __restrict__ ws,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, uint16_t* __restrict__ y) {
    static_assert(U >= 1 && U <= 8, "one scale per lane covers at most 8 steps");
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* xl = lds;
    float* sl = (float*)(lds + K);  // K % 128 == 0 keeps it aligned
    const int64_t nkb = K >> 7;
    const int j = threadIdx.x & 63;
    const int64_t n = first_row<64, 1, WPB>();
    const bool live = n < N;  // wave-uniform
    const uint8_t* wr = w + (live ? n : N - 1) * ldw;
    const int64_t nchunk = K >> 4;
    const int64_t nsteps = (nchunk + 63) >> 6;
    auto load_w = [&](u32x4_t (&wv)[U], int64_t s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * 64 + j;
            wv[u] = ld_stream(wr + (c < nchunk ? c : nchunk - 1) * 16);
        }
    };
    const int64_t ngl = nkb * 16;  // one lane per 8 values (K >= 128: ngl >= 16)
    auto ld_x = [&](int64_t i0) {
        const int64_t i = i0 + threadIdx.x;
        return ld16(x + (i < ngl ? i : ngl - 1) * 8);
    };
    auto quant_pass = [&](int64_t i0, const u32x4_t& v) {
        const int64_t i = i0 + threadIdx.x;
        const bool ok = i < ngl;
        const int64_t g = ok ? (i >> 4) : nkb - 1;
        const int jj = (int)(i & 15);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = bf16_to_f32(d[q] & 0xFFFFu);
            f[2 * q + 1] = bf16_to_f32(d[q] >> 16);
        }
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
        a = row_max_f32(a);  // the 16 lanes of a DPP row hold one group
        const int E = blk_group_exp(a);
        const float sc = blk_group_inv_scale(E);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * sc, f[1] * sc, 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * sc, f[3] * sc, lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * sc, f[5] * sc, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * sc, f[7] * sc, hi, true);
        if (ok) {
            const uint2 c = make_uint2((uint32_t)lo, (uint32_t)hi);
            *(uint2*)(xl + g * 128 + jj * 8) = c;
            if (jj == 0) sl[g] = ue8m0_to_f32((uint32_t)E);
            if ((uint32_t)g % gridDim.x == blockIdx.x) {  // exported only when asked for
                if (xq) *(uint2*)(xq + g * 128 + jj * 8) = c;
                if (xs && jj == 0) xs[g] = (uint8_t)E;
            }
        }
    };
    // the first pass's activations are requested before the weights: loads
    // complete in issue order, so its quantisation runs while the weight
    // batch is still in flight
    const u32x4_t x0 = ld_x(0);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* wsr = ws + ((live ? n : N - 1) >> 7) * nkb;
    auto ld_sw = [&](int64_t s) {  // lane j: weight scale byte of K block s*8 + j
        const int64_t kbl = s * 8 + j;
        return wsr[j < 8 * U && kbl < nkb ? kbl : 0];
    };
    u32x4_t wv[U];
    load_w(wv, 0);
    uint8_t swb = ld_sw(0);
    __builtin_amdgcn_sched_barrier(0);
    quant_pass(0, x0);
    for (int64_t i0 = 64 * WPB; i0 < ngl; i0 += 64 * WPB) quant_pass(i0, ld_x(i0));  // uniform trip count
    __syncthreads();
    if (!live) return;  // no barrier follows

    float acc = 0.0f;
    for (int64_t s = 0; s < nsteps; s += U) {
        if (s > 0) {
            load_w(wv, s);
            swb = ld_sw(s);
        }
        const int64_t kbl = s * 8 + j;
        const bool okb = j < 8 * U && kbl < nkb;
        const float swl = okb ? ue8m0_to_f32(swb) : 0.0f;
        const float sxl = okb ? sl[okb ? kbl : 0] : 0.0f;
        u32x4_t xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (s + u) * 64 + j;
            xv[u] = *(const u32x4_t*)(xl + (c < nchunk ? c : nchunk - 1) * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = (s + u) * 64 + j < nchunk;
            const float sw = __shfl(swl, u * 8 + (j >> 3));
            const float sx = __shfl(sxl, u * 8 + (j >> 3));
            bf16x2_t xb[8], wb[8];
            e4m3x16(xv[u], xb);
            e4m3x16(wv[u], wb);
            float loc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) loc = dot2(wb[i], xb[i], loc);
            acc += ok ? (loc * sx) * sw : 0.0f;  // a lane past the row end adds 0
        }
    }
    acc = group_sum<64>(acc);
    if (j == 0) y[n] = f32_to_bf16(acc);
}

// ------------------------------------------------------------------ one token, activations in LDS
// M = 1 for FP8 weight-only and FP8 W8A8 [Z100 operator-family table, FP8
// row; section 2.2].  A wave owns one weight row and keeps all U of its 1 KB
// steps in flight (lane j reads chunk j + 64u; U <= 8 for W8A8, whose codes
// are widened through registers, U <= 16 for bf16 activations), like the INT8 M = 1
// kernel; the workgroup's WPB waves share one copy of the token row in LDS
// (as bf16), so the activations cost one read per workgroup instead of one
// per row (re-reading them per row from the caches measured ~2 us slower at
// 17408 x 5120).  LDS layout: the first 8 values of chunk c at slot c, the
// last 8 at slot nchunk + c (16 bytes each), so lane j's reads of either half
// are contiguous across the wave.  Staging: bf16 activations go global ->
// LDS with direct loads issued before the weight loads, so the wait for them
// leaves the weights in flight; FP8 activation codes (W8A8) go through
// registers and are widened to bf16 once.  Per lane the chunks are summed in
// order (8 v_dot2 each), then across the wave; epilogue bf16(acc * ws)
// (weight-only) or bf16((acc * xs) * ws) (W8A8), as the other kernels.

template <int W8A8, int U, int WPB, int XF = kFmtE4M3, int WF = kFmtE4M3>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_m1_lds_kernel(
    const void* __restrict__ x, const float* __restrict__ xs, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y) {
    extern __shared__ __align__(16) u32x4_t xl[];  // [2 * nchunk] 16-byte halves
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nchunk = K >> 4, nh = 2 * nchunk;
    // 1. activations (issued first)
    constexpr int NT = 64 * WPB;
    if constexpr (!W8A8) {
        // bf16: one direct load instruction fills 1 KB (64 halves) of LDS
        const uint16_t* xb = (const uint16_t*)x;
        const int ni = (int)((nh + 63) >> 6);
        for (int inst = wv; inst < ni; inst += WPB) {  // wave-uniform
            const int64_t q = (int64_t)inst * 64 + lane, qq = q < nh ? q : nh - 1;
            const int64_t h = qq >= nchunk, c = qq - h * nchunk;
            __builtin_amdgcn_global_load_lds((const void*)(xb + c * 16 + h * 8), (lds_void_t*)(xl + (int64_t)inst * 64),
                                             16, 0, 0);
        }
    }
    // W8A8: each thread widens at most kCodeChunks chunks of codes (K <= 8192)
    constexpr int kCodeChunks = (512 + NT - 1) / NT;
    u32x4_t xc[W8A8 ? kCodeChunks : 1];
    if constexpr (W8A8) {
#pragma unroll
        for (int i = 0; i < kCodeChunks; ++i) {
            const int64_t c = tid + (int64_t)i * NT, cc = c < nchunk ? c : nchunk - 1;
            xc[i] = ld16((const uint8_t*)x + cc * 16);
        }
    }
    // 2. this wave's row, every step in flight
    const int64_t n = (int64_t)blockIdx.x * WPB + wv;
    const int64_t nn = n < N ? n : N - 1;
    const uint8_t* wr = w + nn * ldw;
    u32x4_t wq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = (int64_t)u * 64 + lane, cc = c < nchunk ? c : nchunk - 1;
        wq[u] = ld_stream(wr + cc * 16);
    }
    const float wsv = ws[nn * ws_step];
    // 3. publish the activations: every load issued before the U weight loads
    //    has landed once at most U loads are outstanding
    if constexpr (W8A8) {
#pragma unroll
        for (int i = 0; i < kCodeChunks; ++i) {
            const int64_t c = tid + (int64_t)i * NT;
            if (c < nchunk) {
                bf16x2_t b[8];
                fp8x16<XF>(xc[i], b);
                xl[c] = u32x4_t{__builtin_bit_cast(uint32_t, b[0]), __builtin_bit_cast(uint32_t, b[1]),
                                __builtin_bit_cast(uint32_t, b[2]), __builtin_bit_cast(uint32_t, b[3])};
                xl[nchunk + c] = u32x4_t{__builtin_bit_cast(uint32_t, b[4]), __builtin_bit_cast(uint32_t, b[5]),
                                         __builtin_bit_cast(uint32_t, b[6]), __builtin_bit_cast(uint32_t, b[7])};
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS stores are done
    } else {
        __builtin_amdgcn_s_waitcnt((U & 15) | ((U >> 4) << 14) | 0x70 | 0xF00);  // vmcnt(U)
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();  // not __syncthreads(): that would also wait for the weights
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // The scales are waited for here, under the weight loads: left to
    // itself the compiler sinks their scalar loads into the store's branch,
    // a round trip after the dot product (E4M3 weight-only 17408 x 5120:
    // 14.6 -> 14.5 us per-channel, 14.85 -> 14.6-14.75 us per-tensor).
    const float xsv = W8A8 ? xs[0] : 1.0f;
    asm volatile("" ::"s"(wsv), "s"(xsv));
    // 4. the row's dot product
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = (int64_t)u * 64 + lane;
        const bool ok = c < nchunk;
        const int64_t cc = ok ? c : nchunk - 1;
        bf16x2_t wb[8];
        fp8x16<WF>(wq[u], wb);
        u32x4_t a = xl[cc], b = xl[nchunk + cc];
        if (!ok) a = b = u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = dot2(wb[e], as_bf16x2(a[e]), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = dot2(wb[4 + e], as_bf16x2(b[e]), acc);
    }
    acc = group_sum<64>(acc);
    if (lane == 0 && n < N) {
        const float t = W8A8 ? (acc * xsv) * wsv : acc * wsv;
        y[n] = f32_to_bf16(t);
    }
}

// ------------------------------------------------------------------ E4M3 weight-only, M tokens, rows in LDS
// The one-token kernel above for M tokens (used at M = 2, and with LOOP at
// M = 1 for rows of more than 16 steps) [Z100 operator-family table, FP8
// row; section 2.2]: the workgroup stages the M bf16 token rows once in LDS
// (row m in halves [m * 2 * nchunk, (m + 1) * 2 * nchunk), in the same
// two-half layout), a wave owns one weight row with all U of its 1 KB steps
// in flight, widens each chunk of codes once and dots it with every token
// row; lane m writes token m's output, bf16(acc * ws).  LDS: 2 * M * K
// bytes (whole 1 KB direct-load blocks).  LOOP: rows of more than U steps,
// taken U steps at a time (the next batch loaded after each one).
template <int M, int U, int WPB, bool LOOP = false>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_lds_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, uint16_t* __restrict__ y, int64_t ldy) {
    extern __shared__ __align__(16) u32x4_t xl[];  // [M][2 * nchunk] 16-byte halves
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunk = (int)(K >> 4), nh = 2 * nchunk, nt = M * nh;
    // 1. the token rows (issued first): one direct load instruction fills 1 KB
    //    (64 halves) of LDS; slots past the last half repeat it
    const int ni = (nt + 63) >> 6;
    for (int inst = wv; inst < ni; inst += WPB) {  // wave-uniform
        const int q = inst * 64 + lane, qq = q < nt ? q : nt - 1;
        const int m = qq / nh, r = qq - m * nh;
        const int h = r >= nchunk, c = r - h * nchunk;
        __builtin_amdgcn_global_load_lds((const void*)(x + m * ldx + c * 16 + h * 8),
                                         (lds_void_t*)(xl + (int64_t)inst * 64), 16, 0, 0);
    }
    // 2. this wave's row, every step in flight (LOOP: its first U steps)
    const int64_t n = (int64_t)blockIdx.x * WPB + wv;
    const int64_t nn = n < N ? n : N - 1;
    const uint8_t* wr = w + nn * ldw;
    u32x4_t wq[U];
    auto load_steps = [&](int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (s + u) * 64 + lane, cc = c < nchunk ? c : nchunk - 1;
            wq[u] = ld_stream(wr + (int64_t)cc * 16);
        }
    };
    load_steps(0);
    const float wsv = ws[nn * ws_step];
    // 3. publish the rows: every load issued before the U weight loads has
    //    landed once at most U loads are outstanding
    __builtin_amdgcn_s_waitcnt((U & 15) | ((U >> 4) << 14) | 0x70 | 0xF00);  // vmcnt(U)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();  // not __syncthreads(): that would also wait for the weights
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("" ::"s"(wsv));  // the scale waited for under the weight loads, as in the one-token kernel
    // 4. the row's dot products (LOOP: U steps at a time, the next U loaded
    //    after each batch)
    const int nsteps = LOOP ? (nchunk + 63) >> 6 : U;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
    for (int s = 0;; s += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (s + u) * 64 + lane;
            const bool ok = c < nchunk;
            const int cc = ok ? c : nchunk - 1;
            bf16x2_t wb[8];
            fp8x16<kFmtE4M3>(wq[u], wb);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u32x4_t a = xl[m * nh + cc], b = xl[m * nh + nchunk + cc];
                if (!ok) a = b = u32x4_t{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[m] = dot2(wb[e], as_bf16x2(a[e]), acc[m]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[m] = dot2(wb[4 + e], as_bf16x2(b[e]), acc[m]);
            }
        }
        if (!LOOP || s + U >= nsteps) break;
        load_steps(s + U);
    }
    float out = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float t = group_sum<64>(acc[m]);  // the total in every lane
        out = lane == m ? t : out;
    }
    if (lane < M && n < N) y[lane * ldy + n] = f32_to_bf16(out * wsv);
}

// ------------------------------------------------------------------ INT8, few tokens, codes in LDS
// W8A8 INT8 for M <= 4 tokens [Z100 operator-family table, INT8 row;
// section 2.1].  A wave owns one weight row with all U steps of 1 KB in
// flight (lane j reads chunk j + 64u; U <= 8 with QX, else U <= 16; LOOP:
// longer rows U steps at a time); the workgroup's WPB waves share the M
// token rows of int8 codes in LDS ([m][K] bytes), each chunk dotted with
// v_dot4 (exact int32), summed across the wave, epilogue bf16((acc * xs) *
// ws) then + bias, or the raw sums (out_kind 1).
// QX: the kernel quantises the bf16 token rows itself with the per-token
// rule of the INT8 quantiser (quant8 / absmax8: bit-identical codes and
// scales), so one launch serves the whole layer: every thread loads its
// share of the rows before the weight loads, the per-token absolute maximum
// goes through a wave reduction and one LDS exchange, and each thread
// divides and stores only its own share, all under the weights' HBM
// latency.  Workgroup 0 also writes the codes and scales out when asked.
constexpr int kI8LdsMaxK = 8192;

template <int M, int U, int WPB, bool QX, bool LOOP = false>
__global__ __launch_bounds__(64 * WPB) void gemv_i8_lds_kernel(
    const void* __restrict__ x, int64_t ldx, const float* __restrict__ xs, int xs_step,
    int64_t K, const int8_t* __restrict__ w, int64_t ldw, int64_t N,
    const float* __restrict__ ws, int ws_step, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int out_kind,
    int8_t* __restrict__ xq_out, int64_t ldxq, float* __restrict__ xs_out) {
    extern __shared__ __align__(16) u32x4_t xl[];  // codes [M][K] bytes
    __shared__ float wmax[QX ? WPB : 1][M];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nchunk = K >> 4;
    constexpr int NT = 64 * WPB;
    // 1. activations, issued before the weights
    // 32-bit index math (K <= 8192, M <= 4): the token of a vector or chunk is
    // found by comparisons, not by a 64-bit division ahead of the weight loads
    const int kv = (int)(K >> 3);  // 16-byte bf16 vectors per token row
    auto token_of = [&](int v, int per) {
        int m = 0;
#pragma unroll
        for (int q = 1; q < M; ++q) m += v >= q * per;
        return m;
    };
    constexpr int NV = QX ? (M * (kI8LdsMaxK / 8) + NT - 1) / NT : 1;  // bf16 vectors per thread
    u32x4_t xv[NV];
    const int nvec = M * kv;  // QX: 16-byte bf16 vectors of all M rows
    if constexpr (QX) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NT, vv = v < nvec ? v : nvec - 1;
            const int m = token_of(vv, kv), r = vv - m * kv;
            const u32x4_t t = ld16((const uint16_t*)x + m * ldx + (int64_t)r * 8);
            xv[i] = v < nvec ? t : u32x4_t{0, 0, 0, 0};
        }
    } else {
        const int nc = (int)nchunk, nq = M * nc;
        const int ni = (nq + 63) >> 6;
        for (int inst = wv; inst < ni; inst += WPB) {  // wave-uniform
            const int q = inst * 64 + lane, qq = q < nq ? q : nq - 1;
            const int m = token_of(qq, nc), c = qq - m * nc;
            __builtin_amdgcn_global_load_lds((const void*)((const int8_t*)x + m * ldx + (int64_t)c * 16),
                                             (lds_void_t*)(xl + inst * 64), 16, 0, 0);
        }
    }
    // 2. this wave's row (LOOP: its first U steps)
    static_assert(!(LOOP && QX), "the fused quantiser serves rows of at most U steps");
    const int64_t n = (int64_t)blockIdx.x * WPB + wv;
    const int64_t nn = n < N ? n : N - 1;
    const int8_t* wr = w + nn * ldw;
    u32x4_t wq[U];
    auto load_steps = [&](int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (int64_t)(s + u) * 64 + lane, cc = c < nchunk ? c : nchunk - 1;
            wq[u] = ld_stream(wr + cc * 16);
        }
    };
    load_steps(0);
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quantisation
    // 3. the codes in LDS
    float sc[M];
    if constexpr (QX) {
        float am[M];
#pragma unroll
        for (int m = 0; m < M; ++m) am[m] = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NT;
            const int tok = v < nvec ? token_of(v, kv) : M;  // vectors past the rows are zero
            const float a = absmax8(xv[i], 0.0f);
#pragma unroll
            for (int m = 0; m < M; ++m) am[m] = tok == m ? fmaxf(am[m], a) : am[m];
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float a = row_max_f32(am[m]);
            a = fmaxf(a, __shfl_xor(a, 16));
            a = fmaxf(a, __shfl_xor(a, 32));
            if (lane == 0) wmax[wv][m] = a;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        float amax[M];
        double rc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float a = wmax[0][m];
#pragma unroll
            for (int q = 1; q < WPB; ++q) a = fmaxf(a, wmax[q][m]);
            amax[m] = a;
            sc[m] = a / 127.0f;
            rc[m] = 1.0 / (double)sc[m];
        }
        const bool out = xq_out && blockIdx.x == 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * NT;
            if (v < nvec) {
                const int tok = token_of(v, kv), r = v - tok * kv;
                float a = amax[0];
                double rr = rc[0];
#pragma unroll
                for (int m = 1; m < M; ++m) {
                    a = tok == m ? amax[m] : a;
                    rr = tok == m ? rc[m] : rr;
                }
                const uint2 q = quant8(xv[i], a, rr);
                *(uint2*)((uint8_t*)xl + tok * (int)K + r * 8) = q;
                if (out) *(uint2*)(xq_out + tok * ldxq + (int64_t)r * 8) = q;
            }
        }
        if (xs_out && blockIdx.x == 0 && tid < M) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (tid == m) xs_out[m] = sc[m];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m) sc[m] = xs ? xs[m * xs_step] : 0.0f;
        __builtin_amdgcn_s_waitcnt((U & 15) | ((U >> 4) << 14) | 0x70 | 0xF00);  // vmcnt(U): the direct loads
                                                                                  // have landed
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();  // not __syncthreads(): that would also wait for the weights
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const float wsv = ws ? ws[nn * ws_step] : 0.0f;
    // 4. the row (LOOP: U steps at a time, the next U loaded after each batch)
    const int nsteps = LOOP ? (int)((nchunk + 63) >> 6) : U;
    int acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0;
    for (int s = 0;; s += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = (int64_t)(s + u) * 64 + lane;
            const bool ok = c < nchunk;
            const int64_t cc = ok ? c : nchunk - 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u32x4_t a = xl[m * nchunk + cc];
                if (!ok) a = u32x4_t{0, 0, 0, 0};
                int t = acc[m];
                t = sdot4(wq[u].x, a.x, t);
                t = sdot4(wq[u].y, a.y, t);
                t = sdot4(wq[u].z, a.z, t);
                t = sdot4(wq[u].w, a.w, t);
                acc[m] = t;
            }
        }
        if (!LOOP || s + U >= nsteps) break;
        load_steps(s + U);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = group_sum<64>(acc[m]);
    if (lane == 0 && n < N) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (out_kind == 1) {
                ((int32_t*)y)[m * ldy + n] = acc[m];
            } else {
                float t = (float)acc[m];
                t = t * sc[m];
                t = t * wsv;
                uint16_t o = f32_to_bf16(t);
                if (bias) o = f32_to_bf16(bf16_to_f32(o) + bf16_to_f32(bias[n]));
                ((uint16_t*)y)[m * ldy + n] = o;
            }
        }
    }
}

// ------------------------------------------------------------------ block FP8, one token, activations in LDS
// M = 1 block-scaled FP8 with the activation quantisation fused in [Z100
// section 2.4: block formula, per-block fold; DSV4 section 3.3: per-token
// per-128 E4M3 activations with UE8M0 scales].  The workgroup loads the
// bf16 row first, then every wave issues all U steps of its weight row and
// the row's weight scale bytes; the row is quantised with the rule of
// blk_act_quant_kernel (a 16-lane DPP row per 128-group, exponent from the
// bits of amax, exact power-of-two scaling, RNE convert: bit-identical
// codes), and the decoded code values (exact in bf16) go to LDS in the
// two-half layout of gemv_fp8_m1_lds_kernel, the group scales 2^(E-127) next
// to them.  The barrier after the LDS stores does not wait for the weights,
// so each step's products start as soon as that step's bytes arrive.  Per
// chunk of 16 (inside one 128-block): 8 v_dot2 of widened weights against
// the staged values, then acc += (dot * 2^(xs-127)) * 2^(ws-127), the fold
// order of every block kernel.  Group g goes to xq / xs (each optional) from
// workgroup g % gridDim.x.  Dynamic LDS: 2K bytes of bf16, then K/128 floats.
constexpr int64_t kBlkM1LdsMaxK = 8192;  // U <= 8 steps: a lane holds one K block's weight scale

template <int U, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_fp8_blk_m1_lds_kernel(
    const uint16_t* __restrict__ x, int64_t K,
    const uint8_t* __restrict__ w, int64_t ldw, int64_t N, const uint8_t* __restrict__ ws,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, uint16_t* __restrict__ y) {
    static_assert(U >= 1 && U <= 8, "one scale byte per lane covers at most 8 steps");
    extern __shared__ __align__(16) u32x4_t xl[];  // [2 * nchunk] 16-byte halves of bf16
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunk = (int)(K >> 4), nkb = (int)(K >> 7);
    float* sl = (float*)(xl + 2 * nchunk);
    constexpr int NT = 64 * WPB;
    // 1. the bf16 row: vector i = 8 values, group i / 16; one per thread and pass
    const int nvec = (int)(K >> 3);
    constexpr int kMaxPass = (kBlkM1LdsMaxK / 8 + NT - 1) / NT;
    const int npass = (nvec + NT - 1) / NT;
    u32x4_t xv[kMaxPass];
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        const int i = tid + p * NT;
        xv[p] = p < npass ? ld16(x + (int64_t)(i < nvec ? i : nvec - 1) * 8) : u32x4_t{0, 0, 0, 0};
    }
    // 2. this wave's row: every step and the row's scale bytes
    const int64_t n = (int64_t)blockIdx.x * WPB + wv;
    const int64_t nn = n < N ? n : N - 1;
    const uint8_t* wr = w + nn * ldw;
    u32x4_t wq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = u * 64 + lane;
        wq[u] = ld_stream(wr + (int64_t)(c < nchunk ? c : nchunk - 1) * 16);
    }
    const uint8_t* wsr = ws + (nn >> 7) * nkb;
    const uint8_t swb = wsr[lane < nkb ? lane : nkb - 1];  // lane l: weight scale byte of K block l
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quantisation
    // 3. quantise: the 16 lanes of a DPP row hold the 16 vectors of one group
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        if (p < npass) {  // workgroup-uniform
            const int i = tid + p * NT;
            const bool ok = i < nvec;
            const int g = ok ? (i >> 4) : nkb - 1, jj = i & 15;
            const uint32_t d[4] = {xv[p].x, xv[p].y, xv[p].z, xv[p].w};
            float f[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = bf16_to_f32(d[q] & 0xFFFFu);
                f[2 * q + 1] = bf16_to_f32(d[q] >> 16);
            }
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
            a = row_max_f32(a);
            const int E = blk_group_exp(a);
            const float sc = blk_group_inv_scale(E);
            int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * sc, f[1] * sc, 0, false);
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * sc, f[3] * sc, lo, true);
            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * sc, f[5] * sc, 0, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * sc, f[7] * sc, hi, true);
            if (ok) {
                bf16x2_t b[4];
                e4m3x4_to_bf16((uint32_t)lo, b[0], b[1]);
                e4m3x4_to_bf16((uint32_t)hi, b[2], b[3]);
                // vector i is half (i & 1) of chunk i >> 1
                xl[(i & 1) * nchunk + (i >> 1)] =
                    u32x4_t{__builtin_bit_cast(uint32_t, b[0]), __builtin_bit_cast(uint32_t, b[1]),
                            __builtin_bit_cast(uint32_t, b[2]), __builtin_bit_cast(uint32_t, b[3])};
                if (jj == 0) sl[g] = ue8m0_to_f32((uint32_t)E);
                if ((uint32_t)g % gridDim.x == blockIdx.x) {  // exported only when asked for
                    if (xq) *(uint2*)(xq + (int64_t)i * 8) = make_uint2((uint32_t)lo, (uint32_t)hi);
                    if (xs && jj == 0) xs[g] = (uint8_t)E;
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS stores are done
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();  // not __syncthreads(): that would also wait for the weights
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // 4. the row: chunk c = u*64 + lane lies in K block c / 8
    const float swl = ue8m0_to_f32(swb);
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = u * 64 + lane;
        const bool ok = c < nchunk;
        const int cc = ok ? c : nchunk - 1;
        const float sw = __shfl(swl, cc >> 3);
        const float sx = sl[cc >> 3];
        bf16x2_t wb[8];
        e4m3x16(wq[u], wb);
        const u32x4_t a0 = xl[cc], a1 = xl[nchunk + cc];
        float loc = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) loc = dot2(wb[e], as_bf16x2(a0[e]), loc);
#pragma unroll
        for (int e = 0; e < 4; ++e) loc = dot2(wb[4 + e], as_bf16x2(a1[e]), loc);
        acc += ok ? (loc * sx) * sw : 0.0f;  // a lane past the row end adds 0
    }
    acc = group_sum<64>(acc);
    if (lane == 0 && n < N) y[n] = f32_to_bf16(acc);
}

}  // namespace qlin
