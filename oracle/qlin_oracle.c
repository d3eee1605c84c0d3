/*
 * qlin_oracle.c -- plain, slow CPU oracle for the weight-quantized decode
 * linear layer y[M,N] = dequant(W[N,K]) . x[M,K].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only tests/, the smoke check in __graft_entry__.py and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant generator with the HIP library; the two only see the same inputs.
 *
 * Rules this file follows:
 *   - every function is the plain definition, loop by loop, in the order the
 *     pages state it; no blocking, fusion or reordering;
 *   - floating-point results accumulate in fp64 (double), integer results in
 *     int64, and the final bf16 is produced by one round-to-nearest-even from
 *     the fp64 value;
 *   - the only parallelism is an OpenMP loop over independent output rows,
 *     which does not change any arithmetic;
 *   - compiled with -O2 -ffp-contract=off and without -ffast-math.
 *
 * Sources (web pages, cited by title and section):
 *   [Z100]  "Hygon Z100 (gfx906) vLLM adaptation: optimisation and operator
 *            development record (condensed)", chapter 2 "hand-written HIP
 *            operators": the operator-family table (section 2), and the
 *            subsections 2.1 INT8 W8A8 sdot4, 2.2 FP8 emulation,
 *            2.4 block-scaled (128x128) FP8 extension.
 *   [DSV4]  "vLLM 0.27.x port: DeepSeek V4 Flash FP4 on Hygon DCU gfx936,
 *            full report", section 3.3 (model and quantisation config),
 *            section 7.4 (final reader: UE8M0 decode and worked scale bytes),
 *            section 9.3 (MXFP4 MoE emulation).
 * Where the pages leave a step open, the plainest reading is taken; each
 * reading is marked "READING:" below.
 *
 * Pinned by tests/test_oracle_*.py against values the pages print, closed
 * forms, library routines (torch float8/bf16 casts, numpy matmul), exact
 * rational arithmetic and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Threads                                                                   */
/* ------------------------------------------------------------------------ */

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the top half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* Round a binary32 to bf16, nearest, ties to even (sign-magnitude rounding
 * of the dropped 16 bits).  NaN becomes the canonical quiet NaN 0x7FC0. */
uint16_t orc_f32_to_bf16(float f) {
    if (isnan(f)) return 0x7FC0;
    uint32_t u = f32_bits(f);
    uint16_t hi = (uint16_t)(u >> 16);
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (hi & 1u))) hi += 1; /* may carry into the exponent: correct */
    return hi;
}

/* Round-half-even of a finite double to an integer-valued double. */
static double rne_int(double t) {
    double fl = floor(t);
    double frac = t - fl; /* exact: t and fl share the exponent range */
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Round a double to bf16 with one RNE step (no intermediate float). */
uint16_t orc_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);            /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;           /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;   /* subnormal range has the spacing of 2^-126's binade */
    double spacing = ldexp(1.0, e - 7); /* 8 significant bits */
    double q = rne_int(a / spacing);    /* division by a power of two: exact */
    double mag = q * spacing;
    /* largest finite bf16 = (2 - 2^-7) * 2^127 */
    if (mag > ldexp(255.0, 120)) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (f32_bits((float)mag) >> 16)); /* mag is exactly a bf16 value */
}

/* OCP E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is
 * no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double orc_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9)            /* m/8 * 2^(1-7) */
                          : ldexp((double)(8 + m), e - 10); /* (1+m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* E4M3 encode: round to the nearest finite code, ties to the even mantissa
 * (= even code), saturating to +-448.  READING: the pages do not state the
 * rounding or overflow rule for the activation quantiser; RNE with
 * saturation is the plainest one for a format without infinities.
 * Implemented by plain search over the 127 non-negative finite codes, whose
 * magnitudes increase with the code. */
uint8_t orc_e4m3_encode(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    uint8_t best = 0;
    for (int c = 0; c <= 0x7E; ++c) {
        double lo = orc_e4m3_decode((uint8_t)c);
        if (lo > a) break;
        best = (uint8_t)c; /* largest code with magnitude <= a */
    }
    if (best < 0x7E) {
        double lo = orc_e4m3_decode(best), hi = orc_e4m3_decode((uint8_t)(best + 1));
        double dlo = a - lo, dhi = hi - a;
        if (dhi < dlo || (dhi == dlo && ((best + 1) & 1) == 0)) best = (uint8_t)(best + 1);
    }
    return (uint8_t)(sign | best);
}

/* OCP E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent 0
 * is subnormal (m/4 * 2^-14); exponent 31 holds +-inf (m = 0) and NaN.
 * Largest finite magnitude 57344 (0x7B). */
double orc_e5m2_decode(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 2) & 0x1F, m = c & 3;
    double mag;
    if (e == 31) mag = (m == 0) ? INFINITY : NAN;
    else mag = (e == 0) ? ldexp((double)m, -16)             /* m/4 * 2^(1-15) */
                        : ldexp((double)(4 + m), e - 17);  /* (1+m/4) * 2^(e-15) */
    return s ? -mag : mag;
}

/* E5M2 encode: round to the nearest finite code, ties to the even mantissa
 * (= even code), saturating to +-57344; NaN -> 0x7F.  READING: as for E4M3,
 * RNE with saturation (the quantiser's values never exceed the maximum).
 * Plain search over the 124 non-negative finite codes. */
uint8_t orc_e5m2_encode(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    uint8_t best = 0;
    for (int c = 0; c <= 0x7B; ++c) {
        double lo = orc_e5m2_decode((uint8_t)c);
        if (lo > a) break;
        best = (uint8_t)c;
    }
    if (best < 0x7B) {
        double lo = orc_e5m2_decode(best), hi = orc_e5m2_decode((uint8_t)(best + 1));
        double dlo = a - lo, dhi = hi - a;
        if (dhi < dlo || (dhi == dlo && ((best + 1) & 1) == 0)) best = (uint8_t)(best + 1);
    }
    return (uint8_t)(sign | best);
}

/* OCP E2M1 (MXFP4 element): 1 sign, 2 exponent bits (bias 1), 1 mantissa
 * bit; exponent field 0 is subnormal (m * 0.5). */
double orc_e2m1_decode(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp((double)(2 + m), e - 2); /* (1+m/2)*2^(e-1) */
    return s ? -mag : mag;
}

/* UE8M0 scale byte: 2^(b - 127) [DSV4 section 7.4]; 0xFF encodes NaN. */
double orc_ue8m0_decode(uint8_t b) {
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------------------ */
/* (a) W8A8 INT8 [Z100 section 2 table, INT8 row; section 2.1]              */
/* ------------------------------------------------------------------------ */

/* Dynamic, symmetric, per-token activation quantisation: s = amax/127,
 * q = clamp(round_half_even(x / s), -127, 127), fp32 IEEE arithmetic.
 * READING: amax == 0 gives s = 0 and all codes 0 (the only choice without
 * a 0/0). */
void orc_act_quant_i8(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                      int8_t* xq, int64_t ldxq, float* xs) {
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(orc_bf16_to_f32(x[m * ldx + k]));
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        xs[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int q = 0;
            if (amax != 0.0f) {
                float t = orc_bf16_to_f32(x[m * ldx + k]) / s; /* one fp32 division */
                double r = rne_int((double)t);
                if (r > 127.0) r = 127.0;
                if (r < -127.0) r = -127.0;
                q = (int)r;
            }
            xq[m * ldxq + k] = (int8_t)q;
        }
    }
}

/* acc[m,n] = sum_k xq[m,k] * w[n,k], exact integer accumulation.
 * Epilogue in the order the page gives: (acc * x_s) * w_s in fp32, cast to
 * bf16, then add the bias (if any) in the output type.
 * x_s is [M] or [1]; w_s is [N] or [1] (broadcast). */
void orc_gemv_i8(const int8_t* xq, int64_t ldxq, const float* xs, int xs_per_token,
                 int64_t M, int64_t K, const int8_t* w, int64_t ldw, int64_t N,
                 const float* ws, int ws_per_row, const uint16_t* bias,
                 int32_t* acc_out /* [M][N], nullable */, uint16_t* y, int64_t ldy) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)xq[m * ldxq + k] * (int64_t)w[n * ldw + k];
            if (acc_out) acc_out[m * N + n] = (int32_t)acc;
            float t = (float)acc;
            t = t * xs[xs_per_token ? m : 0];
            t = t * ws[ws_per_row ? n : 0];
            uint16_t out = orc_f32_to_bf16(t);
            if (bias) out = orc_f32_to_bf16(orc_bf16_to_f32(out) + orc_bf16_to_f32(bias[n]));
            y[m * ldy + n] = out;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* (b) FP8-E4M3 weight-only [Z100 section 2 table, FP8 row; section 2.2]    */
/* ------------------------------------------------------------------------ */

/* y[m,n] = ws[n] * sum_k e4m3(w[n,k]) * x[m,k]; the scale is applied once,
 * after the sum.  y_exact (fp64) and S = |ws| * sum_k |w x| are returned for
 * the tolerance check (both nullable). */
void orc_gemv_fp8(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                  const uint8_t* w, int64_t ldw, int64_t N, const float* ws, int ws_per_row,
                  uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        double sc = (double)ws[ws_per_row ? n : 0];
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = orc_e4m3_decode(w[n * ldw + k]) * (double)orc_bf16_to_f32(x[m * ldx + k]);
                acc += p;
                sabs += fabs(p);
            }
            double v = sc * acc;
            y[m * ldy + n] = orc_f64_to_bf16(v);
            if (y_exact) y_exact[m * N + n] = v;
            if (S) S[m * N + n] = fabs(sc) * sabs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 W8A8: e4m3fn or e5m2 codes for both operands, activation scale per   */
/* token or per tensor, weight scale per channel or per tensor              */
/* [Z100 operator-family table, FP8 row (W8A8; e4m3fn/e5m2;                 */
/*  per-tensor/per-channel/per-token); section 2.2 (scale applied once)]    */
/* ------------------------------------------------------------------------ */

#define ORC_FMT_E4M3 0
#define ORC_FMT_E5M2 1

static double orc_fp8_decode(int fmt, uint8_t c) {
    return fmt == ORC_FMT_E5M2 ? orc_e5m2_decode(c) : orc_e4m3_decode(c);
}
static uint8_t orc_fp8_encode(int fmt, double v) {
    return fmt == ORC_FMT_E5M2 ? orc_e5m2_encode(v) : orc_e4m3_encode(v);
}

/* Dynamic activation quantisation: s = amax / fmax (fp32 IEEE division,
 * fmax = 448 for E4M3, 57344 for E5M2), q = encode(fl32(x / s)) with x / s
 * one fp32 division.  amax over the token's row (per_token) or over all M
 * rows (one scale).  READING: the INT8 rule with the format's largest finite
 * value in place of 127; amax == 0 gives s = 0 and zero codes. */
void orc_act_quant_fp8(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, int fmt, int per_token,
                       uint8_t* xq, int64_t ldxq, float* xs) {
    const float fmax = fmt == ORC_FMT_E5M2 ? 57344.0f : 448.0f;
    float gmax = 0.0f;
    if (!per_token)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) {
                float a = fabsf(orc_bf16_to_f32(x[m * ldx + k]));
                if (a > gmax) gmax = a;
            }
    for (int64_t m = 0; m < M; ++m) {
        float amax = gmax;
        if (per_token) {
            amax = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = fabsf(orc_bf16_to_f32(x[m * ldx + k]));
                if (a > amax) amax = a;
            }
        }
        float s = amax / fmax;
        if (per_token || m == 0) xs[per_token ? m : 0] = s;
        for (int64_t k = 0; k < K; ++k) {
            uint8_t q = 0;
            if (amax != 0.0f) {
                float t = orc_bf16_to_f32(x[m * ldx + k]) / s; /* one fp32 division */
                q = orc_fp8_encode(fmt, (double)t);
            }
            xq[m * ldxq + k] = q;
        }
    }
}

/* y = bf16( xs * ws * sum_k dec(xq[m,k]) * dec(w[n,k]) ), the sum and the
 * scaling in fp64; xs is [M] or [1], ws is [N] or [1]. */
void orc_gemv_fp8_w8a8(const uint8_t* xq, int64_t ldxq, const float* xs, int xs_per_token, int x_fmt,
                       int64_t M, int64_t K, const uint8_t* w, int64_t ldw, int64_t N,
                       const float* ws, int ws_per_row, int w_fmt,
                       uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            const double sc = (double)xs[xs_per_token ? m : 0] * (double)ws[ws_per_row ? n : 0];
            double acc = 0.0, sabs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = orc_fp8_decode(x_fmt, xq[m * ldxq + k]) * orc_fp8_decode(w_fmt, w[n * ldw + k]);
                acc += p;
                sabs += fabs(p);
            }
            double v = sc * acc;
            y[m * ldy + n] = orc_f64_to_bf16(v);
            if (y_exact) y_exact[m * N + n] = v;
            if (S) S[m * N + n] = fabs(sc) * sabs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* (c) Block-scaled FP8, 128x128 weight blocks, UE8M0 scales                */
/*     [Z100 section 2.4, block formula and scale-folding identity;         */
/*      DSV4 section 3.3 quantisation config: dynamic activations, e4m3,    */
/*      ue8m0 scale format, 128x128 weight blocks]                          */
/* ------------------------------------------------------------------------ */

#define ORC_BLK 128

/* Per token m and 128-wide K group kb: E = 127 + p with p the smallest
 * integer such that amax <= 448 * 2^p, clamped to [1, 254]; amax == 0 gives
 * E = 127.  Codes: xq = e4m3_encode(x / 2^(E-127)) (division by a power of
 * two is exact).  READING: the pages fix the scale format (UE8M0) and the
 * grouping but not the exponent rule; rounding the scale up to the next
 * power of two is the plainest rule that never overflows E4M3. */
/* Activation quantisation per token and block_k-wide K group (block_k a
 * multiple of 32; 128 in the configuration the pages tested). */
void orc_blk_act_quant_g(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, int64_t bk,
                         uint8_t* xq /* [M][K] */, uint8_t* xs /* [M][K/bk] */) {
    int64_t nkb = K / bk;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            double amax = 0.0;
            for (int64_t k = kb * bk; k < (kb + 1) * bk; ++k) {
                double a = fabs((double)orc_bf16_to_f32(x[m * ldx + k]));
                if (a > amax) amax = a;
            }
            int E = 127;
            if (amax > 0.0) {
                int p = -200;
                while (!(amax <= ldexp(448.0, p))) ++p; /* smallest p with amax <= 448*2^p */
                E = 127 + p;
                if (E < 1) E = 1;
                if (E > 254) E = 254;
            }
            xs[m * nkb + kb] = (uint8_t)E;
            for (int64_t k = kb * bk; k < (kb + 1) * bk; ++k) {
                double v = ldexp((double)orc_bf16_to_f32(x[m * ldx + k]), -(E - 127));
                xq[m * K + k] = orc_e4m3_encode(v);
            }
        }
    }
}

void orc_blk_act_quant(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                       uint8_t* xq /* [M][K] */, uint8_t* xs /* [M][K/128] */) {
    orc_blk_act_quant_g(x, ldx, M, K, ORC_BLK, xq, xs);
}

/* out[m,n] = sum_kb ( sum_{k in kb} xq[m,k] * w[n,k] ) * a_s[m,kb] * w_s[n/128, kb]
 * with every code and scale decoded exactly; ws is [ceil(N/128)][K/128]. */
/* Block-scaled GEMV with block_n x block_k weight blocks (weight scale row
 * n / block_n) and block_k-wide activation groups: per K block the two
 * power-of-two scales multiply that block's exact partial sum [Z100 section
 * 2.4: block formula; block_n, block_k runtime parameters, block_k % 32]. */
void orc_gemv_fp8_blk_g(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                        const uint8_t* w, int64_t ldw, int64_t N, const uint8_t* ws, int64_t bn, int64_t bk,
                        uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    int64_t nkb = K / bk;
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double tot = 0.0, sabs = 0.0;
            for (int64_t kb = 0; kb < nkb; ++kb) {
                double part = 0.0, pabs = 0.0;
                for (int64_t k = kb * bk; k < (kb + 1) * bk; ++k) {
                    double p = orc_e4m3_decode(xq[m * K + k]) * orc_e4m3_decode(w[n * ldw + k]);
                    part += p;
                    pabs += fabs(p);
                }
                double sc = orc_ue8m0_decode(xs[m * nkb + kb]) * orc_ue8m0_decode(ws[(n / bn) * nkb + kb]);
                tot += part * sc;
                sabs += pabs * fabs(sc);
            }
            y[m * ldy + n] = orc_f64_to_bf16(tot);
            if (y_exact) y_exact[m * N + n] = tot;
            if (S) S[m * N + n] = sabs;
        }
    }
}

void orc_gemv_fp8_blk(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                      const uint8_t* w, int64_t ldw, int64_t N, const uint8_t* ws,
                      uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    orc_gemv_fp8_blk_g(xq, xs, M, K, w, ldw, N, ws, ORC_BLK, ORC_BLK, y, ldy, y_exact, S);
}

/* ------------------------------------------------------------------------ */
/* (d) MXFP4 expert GEMV behind top-k routing [DSV4 section 9.3; the       */
/*     MXFP4 element/scale formats of the OCP MX spec: E2M1 elements, one   */
/*     UE8M0 scale per 32 K-elements]                                       */
/* ------------------------------------------------------------------------ */

/* y[t,n] = sum_j g[t,j] * sum_k e2m1(W[e,n,k]) * 2^(S[e,n,k/32]-127) * x[t,k],
 * e = ids[t,j].  READING: W is [E][N][K/2] bytes with element 2i in the low
 * nibble of byte i; S is [E][N][K/32]; an id outside [0, E) contributes 0;
 * the op is gather -> per-expert GEMV -> weighted sum (no activation). */
void orc_moe_mxfp4(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                   const uint8_t* w, const uint8_t* s, int64_t E, int64_t N,
                   const int32_t* ids, const float* gw, int64_t topk,
                   uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t t = 0; t < M; ++t) {
            double tot = 0.0, sabs = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                int64_t e = ids[t * topk + j];
                if (e < 0 || e >= E) continue;
                double g = (double)gw[t * topk + j];
                const uint8_t* wrow = w + (e * N + n) * (K / 2);
                const uint8_t* srow = s + (e * N + n) * (K / 32);
                double dot = 0.0, dabs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    uint8_t byte = wrow[k / 2];
                    uint8_t nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                    double p = orc_e2m1_decode(nib) * orc_ue8m0_decode(srow[k / 32]) *
                               (double)orc_bf16_to_f32(x[t * ldx + k]);
                    dot += p;
                    dabs += fabs(p);
                }
                tot += g * dot;
                sabs += fabs(g) * dabs;
            }
            y[t * ldy + n] = orc_f64_to_bf16(tot);
            if (y_exact) y_exact[t * N + n] = tot;
            if (S) S[t * N + n] = sabs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MoE expert FFN with on-device routing: router logits -> top-k -> softmax  */
/* over the selected logits -> per routed pair gate/up MXFP4 GEMVs ->        */
/* clamped SwiGLU -> down MXFP4 GEMV -> weighted sum [DSV4 section 9.3 (the  */
/* MXFP4 expert path), sections 6.6 (J09) and 9.4 (SwiGLU with alpha 1.0,    */
/* limit 10.0)].                                                              */
/* ------------------------------------------------------------------------ */

/* logit[m][e] = sum_k x[m][k] * wr[e][k], bf16 inputs, fp64 sum.
 * READING: the router is a plain bf16 linear layer without bias; the pages
 * name the routing fast path but not its scoring function. */
void orc_router_logits(const uint16_t* x, int64_t ldx, int64_t M, int64_t H,
                       const uint16_t* wr, int64_t E, double* logits) {
    int64_t e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < E; ++e) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < H; ++k)
                acc += (double)orc_bf16_to_f32(x[m * ldx + k]) * (double)orc_bf16_to_f32(wr[e * H + k]);
            logits[m * E + e] = acc;
        }
    }
}

/* The k largest logits of each token, largest first.
 * READING: equal logits go to the lower expert id (the first one met). */
void orc_topk(const double* logits, int64_t M, int64_t E, int64_t k, int32_t* ids) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int64_t q = 0; q < j; ++q) taken |= ids[m * k + q] == e;
                if (taken) continue;
                if (best < 0 || logits[m * E + e] > logits[m * E + best]) best = e;
            }
            ids[m * k + j] = (int32_t)best;
        }
    }
}

/* Routing weights: softmax over the selected experts' logits.
 * READING: renormalised over the top-k (as the routing weights of the
 * expert GEMV are). */
void orc_topk_softmax(const double* logits, int64_t M, int64_t E, const int32_t* ids, int64_t k,
                      double* g) {
    for (int64_t m = 0; m < M; ++m) {
        double mx = -INFINITY, den = 0.0;
        for (int64_t j = 0; j < k; ++j) mx = fmax(mx, logits[m * E + ids[m * k + j]]);
        for (int64_t j = 0; j < k; ++j) den += exp(logits[m * E + ids[m * k + j]] - mx);
        for (int64_t j = 0; j < k; ++j) g[m * k + j] = exp(logits[m * E + ids[m * k + j]] - mx) / den;
    }
}

/* silu(alpha * min(gate, limit)) * clamp(up, -limit, limit), silu(z) = z / (1 + e^-z). */
double orc_swiglu(double gate, double up, double alpha, double limit) {
    const double gc = gate > limit ? limit : gate;
    const double uc = up > limit ? limit : (up < -limit ? -limit : up);
    const double z = alpha * gc;
    return z / (1.0 + exp(-z)) * uc;
}

void orc_swiglu_n(const double* gate, const double* up, int64_t n, double alpha, double limit, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_swiglu(gate[i], up[i], alpha, limit);
}

/* One MXFP4 row (E2M1 codes, element 2i in the low nibble of byte i, one
 * UE8M0 scale per 32) dotted with a bf16 vector of length K, fp64. */
static double orc_mxfp4_row_dot(const uint8_t* wrow, const uint8_t* srow, const uint16_t* v, int64_t K,
                                double* abs_sum) {
    double dot = 0.0, dabs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        uint8_t byte = wrow[k / 2];
        uint8_t nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        double p = orc_e2m1_decode(nib) * orc_ue8m0_decode(srow[k / 32]) * (double)orc_bf16_to_f32(v[k]);
        dot += p;
        dabs += fabs(p);
    }
    if (abs_sum) *abs_sum = dabs;
    return dot;
}

/* Expert FFN for a given routing (ids [M][k], weights g [M][k]):
 *   gate = W13[e] rows 0..I-1 . x[t],  up = W13[e] rows I..2I-1 . x[t]
 *   act[p][i] = bf16(swiglu(gate_i, up_i))        (p = t*k + j)
 *   out[p][h] = W2[e] row h . act[p]
 *   y[t][h]   = bf16(sum_j g[t][j] * out[p][h]),  S = sum_j |g| sum_i |w2 * act|
 * w13 [E][2I][H/2], s13 [E][2I][H/32], w2 [E][H][I/2], s2 [E][H][I/32].
 * READING: gate and up are fp32-or-better sums and the activation is rounded
 * once to bf16, the input type of the down projection. */
void orc_moe_ffn_mxfp4(const uint16_t* x, int64_t ldx, int64_t M, int64_t H,
                       const uint8_t* w13, const uint8_t* s13, const uint8_t* w2, const uint8_t* s2,
                       int64_t E, int64_t I, const int32_t* ids, const double* g, int64_t k,
                       double alpha, double limit, uint16_t* act,
                       uint16_t* y, int64_t ldy, double* y_exact, double* S) {
    const int64_t P = M * k;
    int64_t pi;
#pragma omp parallel for schedule(static)
    for (pi = 0; pi < P * I; ++pi) {
        const int64_t p = pi / I, i = pi % I, t = p / k;
        const int64_t e = ids[p];
        if (e < 0 || e >= E) { act[p * I + i] = 0; continue; }
        const double gate = orc_mxfp4_row_dot(w13 + (e * 2 * I + i) * (H / 2), s13 + (e * 2 * I + i) * (H / 32),
                                              x + t * ldx, H, NULL);
        const double up = orc_mxfp4_row_dot(w13 + (e * 2 * I + I + i) * (H / 2),
                                            s13 + (e * 2 * I + I + i) * (H / 32), x + t * ldx, H, NULL);
        act[p * I + i] = orc_f64_to_bf16(orc_swiglu(gate, up, alpha, limit));
    }
    int64_t h;
#pragma omp parallel for schedule(static)
    for (h = 0; h < H; ++h) {
        for (int64_t t = 0; t < M; ++t) {
            double tot = 0.0, sabs = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                const int64_t p = t * k + j, e = ids[p];
                if (e < 0 || e >= E) continue;
                double dabs;
                const double dot = orc_mxfp4_row_dot(w2 + (e * H + h) * (I / 2), s2 + (e * H + h) * (I / 32),
                                                     act + p * I, I, &dabs);
                tot += g[p] * dot;
                sabs += fabs(g[p]) * dabs;
            }
            y[t * ldy + h] = orc_f64_to_bf16(tot);
            if (y_exact) y_exact[t * H + h] = tot;
            if (S) S[t * H + h] = sabs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the format helpers (loops over the scalar routines).      */
/* ------------------------------------------------------------------------ */

void orc_f64_to_bf16_n(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(v[i]);
}

void orc_f32_to_bf16_n(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(v[i]);
}

void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

void orc_e5m2_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_decode(c[i]);
}

void orc_e5m2_encode_n(const double* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode(v[i]);
}

void orc_e4m3_encode_n(const double* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}
