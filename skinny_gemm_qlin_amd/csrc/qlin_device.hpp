// qlin_device.hpp -- device-side helpers shared by the gfx950 kernels.
//
// Number formats decoded here (the kernels never build lookup tables):
//   bf16   top half of an IEEE binary32;
//   E4M3   OCP fp8 (bias 7, no infinities, max 448), converted by the
//          gfx950 hardware converts v_cvt_scalef32_pk_bf16_fp8 /
//          v_cvt_pk_fp8_f32;
//   E5M2   OCP bf8 (bias 15, max 57344), v_cvt_scalef32_pk_bf16_bf8 /
//          v_cvt_pk_bf8_f32;
//   E2M1   OCP fp4 element, converted by v_cvt_scalef32_pk_bf16_fp4;
//   UE8M0  scale byte b meaning 2^(b-127) (byte 255 = NaN), built directly
//          as fp32 bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

// LDS destination of the buffer / global loads that write LDS directly
typedef __attribute__((address_space(3))) void lds_void_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kGroup = 16;  // lanes that share one weight row (one DPP row)

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// UE8M0 byte -> fp32 scale 2^(b-127).  b = 0 is the fp32 subnormal 2^-127,
// b = 255 is NaN.  Selects, not branches (the compiler would otherwise put an
// exec-mask branch around every scale in a kernel's inner loop).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
    uint32_t u = b << 23;
    u = b == 0u ? 0x00400000u : u;
    u = b == 255u ? 0x7FC00000u : u;
    return __uint_as_float(u);
}

// UE8M0 exponent byte of an activation group whose absolute maximum is amax:
// E = 127 + p for the smallest integer p with amax <= 448 * 2^p, clamped to
// [1, 254]; amax = 0 gives 127 [DSV4 section 3.3: power-of-two block scales;
// Z100 section 2.4].  With amax = (1 + f) * 2^(e-127), 448 = 1.75 * 2^8 gives
// p = e - 135 when 1 + f <= 1.75 and e - 134 otherwise; a subnormal amax
// (e = 0) lands below 1 and clamps to 1.
__device__ __forceinline__ int blk_group_exp(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    const int ex = (int)(bits >> 23);
    int E = ex - (((bits & 0x7FFFFFu) <= 0x600000u) ? 8 : 7);
    E = E < 1 ? 1 : (E > 254 ? 254 : E);
    return amax == 0.0f ? 127 : E;
}

// 2^(127 - E) for E in [1, 254], the factor that maps a group onto the E4M3
// range (E = 254 gives the fp32 subnormal 2^-127; every product stays exact
// wherever the E4M3 rounding can see it).
__device__ __forceinline__ float blk_group_inv_scale(int E) {
    const int inv = 254 - E;
    return inv == 0 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)inv << 23);
}

// Four E4M3 codes (one dword) -> two bf16 pairs, exact (E4M3 embeds in bf16).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t d, bf16x2_t& lo, bf16x2_t& hi) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true);
}

// FP8 code formats of the W8A8 path (values of the C ABI's fmt arguments).
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE5M2 = 1;

// Four FP8 codes of format F -> two bf16 pairs, exact (both formats embed in
// bf16: at most 3 mantissa bits, exponents within bf16's normal range).
template <int F>
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t d, bf16x2_t& lo, bf16x2_t& hi) {
    if constexpr (F == kFmtE5M2) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d, 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d, 1.0f, true);
    } else {
        e4m3x4_to_bf16(d, lo, hi);
    }
}

// Two fp32 values -> two FP8 codes of format F (round to nearest even) in
// the low (HI = false) or high 16 bits of `old`.
template <int F, bool HI>
__device__ __forceinline__ int f32x2_to_fp8(float a, float b, int old) {
    if constexpr (F == kFmtE5M2) return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    else return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) ->
// four bf16 pairs, exact.
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t d, bf16x2_t out[4]) {
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0);
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1);
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2);
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------------------- DPP reductions
// DPP row = 16 lanes.  row_ror:n (control 0x120 + n) rotates a row by n lanes;
// v + ror(v,8) + ror(.,4) + ror(.,2) + ror(.,1) leaves the row sum in every
// lane of the row.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ int row_sum_i32(int v) {
    v += dpp_mov<0x128>(v);
    v += dpp_mov<0x124>(v);
    v += dpp_mov<0x122>(v);
    v += dpp_mov<0x121>(v);
    return v;
}

__device__ __forceinline__ float row_sum_f32(float v) {
    v += __int_as_float(dpp_mov<0x128>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x124>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x122>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x121>(__float_as_int(v)));
    return v;
}

__device__ __forceinline__ float row_max_f32(float v) {
    v = fmaxf(v, __int_as_float(dpp_mov<0x128>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<0x124>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<0x122>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<0x121>(__float_as_int(v))));
    return v;
}

// 16-byte global load of read-once weight data (non-temporal hint).
__device__ __forceinline__ u32x4_t ld_stream(const void* p) {
    return __builtin_nontemporal_load((const u32x4_t*)p);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }

// ---------------------------------------------------------------- INT8 activation quantisation
// The per-token rule [Z100 section 2.1; operator-family table, INT8 row]:
// s = amax / 127 (IEEE fp32 division: the build asks for correctly rounded
// division), q = clamp(rne(x / s), -127, 127) with x / s the IEEE fp32
// quotient, q = 0 when amax = 0.
// Shared by the standalone quantiser and the GEMVs that quantise their own
// activations, so their codes are bit-identical.

// The fp32 quotient x / s without a division: with r = fl64(1 / s) (one
// correctly rounded fp64 division per token), fl32(fl64(x * r)) equals the
// IEEE fp32 division fl32(x / s) for fp32 x and s.  Proof: t = fl64(x * r)
// is within about 2^-52 |x/s| of x/s.  A quotient of two 24-bit significands
// is never exactly an fp32 rounding midpoint (a midpoint has an odd 25-bit
// significand, and x = B * s would give x more than 24 bits), and for any
// midpoint B, x - B*s is a nonzero multiple of a power-of-two grid that keeps
// x/s at least 2^-49 |B| away from B; so t and x/s lie on the same side of
// every midpoint and round to the same fp32 value.  (Checked exhaustively
// over every positive bf16 x for 1,200 scales in the CPU tests.)  The fp64
// multiply and the two converts replace a ~10-instruction divide.
__device__ __forceinline__ float div_bf16(float x, double r) { return (float)((double)x * r); }

// 8 bf16 (one 16-byte vector) -> 8 int8 codes (8 bytes, element order kept);
// r = fl64(1 / s).
__device__ __forceinline__ uint2 quant8(const u32x4_t& v, float amax, double r) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = (e & 1) ? (d[e >> 1] >> 16) : (d[e >> 1] & 0xFFFFu);
        int q = 0;
        if (amax != 0.0f) {
            float t = rintf(div_bf16(bf16_to_f32(h), r));
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            q = (int)t;
        }
        packed[e >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (e & 3));
    }
    return make_uint2(packed[0], packed[1]);
}

// max(a, |x|) over 8 bf16 values.
__device__ __forceinline__ float absmax8(const u32x4_t& v, float a) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a = fmaxf(a, fabsf(bf16_to_f32(d[q] & 0xFFFFu)));
        a = fmaxf(a, fabsf(bf16_to_f32(d[q] >> 16)));
    }
    return a;
}

}  // namespace qlin
