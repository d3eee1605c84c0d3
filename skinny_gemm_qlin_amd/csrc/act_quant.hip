// act_quant.hip -- activation quantisers for gfx950.
//
//   act_quant_i8_kernel   per-token symmetric INT8: s = amax/127, q = rne(x/s)
//                         [Z100 section 2.1; operator-family table, INT8 row]
//   blk_act_quant_kernel  per (token, 128-wide K group) E4M3 codes with a
//                         UE8M0 exponent [DSV4 section 3.3; Z100 section 2.4]
//   blkg_act_quant_kernel the same per (token, block_k-wide group), any
//                         block_k that is a multiple of 32 [Z100 section 2.4]
//   act_quant_fp8_kernel  per-token or per-tensor E4M3 / E5M2 codes with an
//                         fp32 scale amax/fmax [Z100 operator-family table,
//                         FP8 row: W8A8, e4m3fn/e5m2, per-token/per-tensor]
#include "qlin_device.hpp"
#include "qlin_launch.hpp"

namespace qlin {

// One workgroup (512 lanes) per token.  Pass 1: amax over the row with
// 16-byte loads (the first kCached vectors of each lane stay in registers);
// DPP row max, then across the 4 rows of a wave, then across the 8 waves
// through LDS.  Pass 2: the IEEE fp32 quotient x / s (div_bf16) and
// round-half-even (v_rndne_f32), clamp to +-127, 8 codes per 8-byte store.  512 lanes rather
// than 256 halve the divisions on each lane's path (2.74 -> 2.30 us per
// 5120-wide token on MI355X, codes unchanged).
constexpr int kQuantThreads = 512;
constexpr int kCached = 2;  // K <= 8192 is read from HBM exactly once

__global__ __launch_bounds__(kQuantThreads) void act_quant_i8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
    int8_t* __restrict__ xq, int64_t ldxq, float* __restrict__ xs) {
    constexpr int W = kQuantThreads / 64;
    __shared__ float wave_max[W];
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    const int tid = threadIdx.x;
    const int64_t nvec = K >> 3;  // 8 bf16 per 16-byte vector

    u32x4_t cache[kCached];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int64_t i = tid + c * kQuantThreads;
        cache[c] = i < nvec ? ld16(row + i * 8) : u32x4_t{0, 0, 0, 0};
        a = absmax8(cache[c], a);
    }
    for (int64_t i = tid + kCached * kQuantThreads; i < nvec; i += kQuantThreads) a = absmax8(ld16(row + i * 8), a);
    a = row_max_f32(a);
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    if ((tid & 63) == 0) wave_max[tid >> 6] = a;
    __syncthreads();
    float amax = wave_max[0];
#pragma unroll
    for (int q = 1; q < W; ++q) amax = fmaxf(amax, wave_max[q]);
    const float s = amax / 127.0f;
    if (tid == 0) xs[m] = s;
    const double r = 1.0 / (double)s;  // x / s per element as div_bf16(x, r)

    int8_t* qrow = xq + m * ldxq;
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int64_t i = tid + c * kQuantThreads;
        if (i < nvec) *(uint2*)(qrow + i * 8) = quant8(cache[c], amax, r);
    }
    for (int64_t i = tid + kCached * kQuantThreads; i < nvec; i += kQuantThreads)
        *(uint2*)(qrow + i * 8) = quant8(ld16(row + i * 8), amax, r);
}

hipError_t launch_act_quant_i8(const ActQuantI8Args& a, hipStream_t st) {
    hipLaunchKernelGGL(act_quant_i8_kernel, dim3((unsigned)a.M), dim3(kQuantThreads), 0, st,
                       a.x, a.ldx, a.K, a.xq, a.ldxq, a.xs);
    return hipGetLastError();
}

// One wavefront per 4 groups of 128: a 16-lane DPP row owns one group, each
// lane 8 consecutive values (one 16-byte load).  E follows from the bits of
// amax = (1+f)*2^e: amax <= 448*2^p = 1.75*2^(p+8) gives p = e-8 when
// 1+f <= 1.75 (mantissa bits <= 0x600000), else p = e-7.  Scaling by
// 2^(127-E) is exact; v_cvt_pk_fp8_f32 rounds to nearest even.
__global__ __launch_bounds__(64) void blk_act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int64_t m = blockIdx.y;
    const int64_t nkb = K >> 7;
    const int64_t kb = (int64_t)blockIdx.x * 4 + g;
    const bool ok = kb < nkb;
    const int64_t kbc = ok ? kb : nkb - 1;

    u32x4_t v = ld16(x + m * ldx + kbc * 128 + j * 8);
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
    a = row_max_f32(a);

    const int E = blk_group_exp(a);
    const float sc = blk_group_inv_scale(E);

    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * sc, f[1] * sc, lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * sc, f[3] * sc, lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * sc, f[5] * sc, hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * sc, f[7] * sc, hi, true);
    if (ok) {
        *(uint2*)(xq + m * K + kb * 128 + j * 8) = make_uint2((uint32_t)lo, (uint32_t)hi);
        if (j == 0) xs[m * nkb + kb] = (uint8_t)E;
    }
}

// ---------------------------------------------------------------- FP8 W8A8
// The INT8 rule with the format's largest finite value fmax (448 for E4M3,
// 57344 for E5M2) in place of 127: s = amax / fmax and q = rne(x / s), both
// IEEE fp32 quotients (x / s formed by div_bf16, the same bits).  |x / s| can exceed fmax by a rounding error (and by
// more when s is an fp32 subnormal); such values saturate to +-fmax before
// the convert, so every code is finite.  The comparisons keep a NaN (which
// then converts to a NaN code).  amax == 0 gives s = 0 and zero codes.
template <int F>
__device__ __forceinline__ uint2 quant_fp8x8(const u32x4_t& v, float amax, double r) {
    constexpr float fmax = F == kFmtE5M2 ? 57344.0f : 448.0f;
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = (e & 1) ? (d[e >> 1] >> 16) : (d[e >> 1] & 0xFFFFu);
        float q = 0.0f;
        if (amax != 0.0f) {
            q = div_bf16(bf16_to_f32(h), r);  // the IEEE fp32 quotient x / s, r = fl64(1 / s)
            q = q > fmax ? fmax : (q < -fmax ? -fmax : q);
        }
        t[e] = q;
    }
    int lo = 0, hi = 0;
    lo = f32x2_to_fp8<F, false>(t[0], t[1], lo);
    lo = f32x2_to_fp8<F, true>(t[2], t[3], lo);
    hi = f32x2_to_fp8<F, false>(t[4], t[5], hi);
    hi = f32x2_to_fp8<F, true>(t[6], t[7], hi);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// One workgroup of T lanes quantises `rows` consecutive tokens with one
// scale: rows = 1 and a grid of M workgroups for per-token scales, rows = M
// and a single workgroup for the per-tensor scale.  The rows' 16-byte
// vectors are numbered row-major; lane l takes vectors l, l + T, ...; the
// first C of them stay in registers between the amax pass and the quantise
// pass (M*K <= 8*T*C values are read from HBM once).  The amax is reduced
// with DPP within a 16-lane row, shuffles across a wave and LDS across waves.
template <int F, int T, int C, bool ONE_ROW>
__global__ __launch_bounds__(T) void act_quant_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int rows_arg, int64_t K,
    uint8_t* __restrict__ xq, int64_t ldxq, float* __restrict__ xs) {
    const int rows = ONE_ROW ? 1 : rows_arg;  // per-token: no row split of the vector index
    constexpr int W = T / 64;
    constexpr float fmax = F == kFmtE5M2 ? 57344.0f : 448.0f;
    __shared__ float wave_max[W];
    const int64_t m0 = (int64_t)blockIdx.x * rows;
    const int tid = threadIdx.x;
    const int nvec = (int)(K >> 3);  // 8 bf16 per vector
    const int total = rows * nvec;

    u32x4_t cache[C];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int i = tid + c * T;
        if (i < total) {
            const int r = ONE_ROW ? 0 : i / nvec, v = i - r * nvec;
            cache[c] = ld16(x + (m0 + r) * ldx + (int64_t)v * 8);
        } else {
            cache[c] = u32x4_t{0, 0, 0, 0};
        }
        a = absmax8(cache[c], a);
    }
    for (int i = tid + C * T; i < total; i += T) {
        const int r = ONE_ROW ? 0 : i / nvec, v = i - r * nvec;
        a = absmax8(ld16(x + (m0 + r) * ldx + (int64_t)v * 8), a);
    }
    a = row_max_f32(a);
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    if ((tid & 63) == 0) wave_max[tid >> 6] = a;
    __syncthreads();
    float amax = wave_max[0];
#pragma unroll
    for (int q = 1; q < W; ++q) amax = fmaxf(amax, wave_max[q]);
    const float s = amax / fmax;
    if (tid == 0) xs[blockIdx.x] = s;
    const double rs = 1.0 / (double)s;

#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int i = tid + c * T;
        if (i < total) {
            const int r = ONE_ROW ? 0 : i / nvec, v = i - r * nvec;
            *(uint2*)(xq + (m0 + r) * ldxq + (int64_t)v * 8) = quant_fp8x8<F>(cache[c], amax, rs);
        }
    }
    for (int i = tid + C * T; i < total; i += T) {
        const int r = ONE_ROW ? 0 : i / nvec, v = i - r * nvec;
        *(uint2*)(xq + (m0 + r) * ldxq + (int64_t)v * 8) =
            quant_fp8x8<F>(ld16(x + (m0 + r) * ldx + (int64_t)v * 8), amax, rs);
    }
}

template <int F>
hipError_t launch_act_quant_fp8_fmt(const ActQuantF8Args& a, hipStream_t st) {
    if (a.per_token)
        hipLaunchKernelGGL((act_quant_fp8_kernel<F, kQuantThreads, kCached, true>), dim3((unsigned)a.M),
                           dim3(kQuantThreads), 0, st, a.x, a.ldx, 1,
                           a.K, a.xq, a.ldxq, a.xs);
    else
        hipLaunchKernelGGL((act_quant_fp8_kernel<F, 1024, 16, false>), dim3(1), dim3(1024), 0, st, a.x, a.ldx, (int)a.M,
                           a.K, a.xq, a.ldxq, a.xs);
    return hipGetLastError();
}

hipError_t launch_act_quant_fp8(const ActQuantF8Args& a, hipStream_t st) {
    return a.fmt == kFmtE5M2 ? launch_act_quant_fp8_fmt<kFmtE5M2>(a, st) : launch_act_quant_fp8_fmt<kFmtE4M3>(a, st);
}

// Any block_k (a multiple of 32): one workgroup per token, one lane per
// K group (groups g, g + 256, ...).  Pass 1 takes the group's amax with
// 16-byte loads, pass 2 re-reads the group (a cache hit) and converts
// x * 2^(127-E) to E4M3 (exact scaling, RNE convert); E follows the same
// rule as blk_act_quant_kernel.
__global__ __launch_bounds__(256) void blkg_act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t K, int64_t bk,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    const int64_t m = blockIdx.x;
    const int64_t nkb = K / bk;
    const uint16_t* row = x + m * ldx;
    for (int64_t g = threadIdx.x; g < nkb; g += 256) {
        float a = 0.0f;
        for (int64_t v = 0; v < bk; v += 8) a = absmax8(ld16(row + g * bk + v), a);
        const int E = blk_group_exp(a);
        const float sc = blk_group_inv_scale(E);
        xs[m * nkb + g] = (uint8_t)E;
        for (int64_t v = 0; v < bk; v += 8) {
            const u32x4_t d = ld16(row + g * bk + v);
            const uint32_t w[4] = {d.x, d.y, d.z, d.w};
            float f[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = bf16_to_f32(w[q] & 0xFFFFu) * sc;
                f[2 * q + 1] = bf16_to_f32(w[q] >> 16) * sc;
            }
            int lo = 0, hi = 0;
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], lo, false);
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], hi, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
            *(uint2*)(xq + m * K + g * bk + v) = make_uint2((uint32_t)lo, (uint32_t)hi);
        }
    }
}

hipError_t launch_blkg_act_quant(const BlkQuantArgs& a, int64_t bk, hipStream_t st) {
    hipLaunchKernelGGL(blkg_act_quant_kernel, dim3((unsigned)a.M), dim3(256), 0, st, a.x, a.ldx, a.K, bk, a.xq, a.xs);
    return hipGetLastError();
}

hipError_t launch_blk_act_quant(const BlkQuantArgs& a, hipStream_t st) {
    const int64_t nkb = a.K >> 7;
    dim3 grid((unsigned)((nkb + 3) / 4), (unsigned)a.M);
    hipLaunchKernelGGL(blk_act_quant_kernel, grid, dim3(64), 0, st, a.x, a.ldx, a.K, a.xq, a.xs);
    return hipGetLastError();
}

}  // namespace qlin
