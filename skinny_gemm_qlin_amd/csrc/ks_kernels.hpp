// ks_kernels.hpp -- K-slice matrix-core decode kernels for gfx950: one
// workgroup per compute unit, each wave owning a fixed slice of K (see below).
#pragma once
#include <type_traits>

#include "mfma_kernels.hpp"

namespace qlin {

// ------------------------------------------------------------------ K-slice kernels (decode shapes)
// For K a multiple of 1024 the dense decode paths (INT8, E4M3 weight-only,
// FP8 W8A8 in its four format pairs) also have kernels laid out for the whole chip rather than
// for one row tile.  The grid holds one workgroup per compute unit (fewer when
// N is small); workgroup b owns the runs of 4 rows b, b + G, b + 2G, ...
// (row j of the workgroup is n = 4*((j/4)*G + b) + j%4, j < R, so that no
// workgroup has more than one run above another and a lane's 4 output rows
// are adjacent), or in one of two other layouts (LAYOUT below), taken as T
// tiles of 16 (in npass passes of T tiles when a workgroup has more rows).  Each of its 8 waves owns one eighth of K (L lines of 128
// bytes) for the whole kernel: it loads its slice of the M token rows once,
// into registers in the MFMA B layout (one-byte codes from 4 tokens on
// through an LDS stage, see XS below), then streams its slice of the T weight
// tiles with the following tiles' loads in flight (8 rows x 128 bytes per
// load instruction), transposing each 128-byte line of a tile through a
// 16-row LDS column into the MFMA A layout.  The 8 partial tiles are summed in
// wave order after one barrier (deterministic; exact for INT8).  Against one
// workgroup per 16-row tile, the activations are read once per wave instead
// of once per tile, and no compute unit is left with an extra tile.  The tile
// loop is unrolled at compile time and no load sits under a branch, so the
// compiler's load counters stay exact and each wait covers one tile only.
constexpr int kKsI8 = 0;      // INT8 codes x INT8 codes, int32 sums
constexpr int kKsF8 = 1;      // E4M3 weights x bf16 activations, fp32 sums
constexpr int kKsW8A8 = 2;    // FP8 weights (WF) x FP8 activation codes (XF), fp32 sums
constexpr int kKsWaves = 8;   // waves per workgroup = K slices
// Row layouts (runs = ceil(N/4) runs of 4 rows; G workgroups)
constexpr int kKsTurn = 0;    // the runs dealt out in turn: workgroup b takes runs b, b + G, ...
constexpr int kKsBlocks = 1;  // G contiguous blocks of floor(runs/G) runs or one more (the first runs mod G)
constexpr int kKsBands = 2;   // whole 16-row tiles dealt out in turn (floor(runs/4G) each), then the
                              // remaining runs in turn
constexpr int kKsMaxTiles = 6;
constexpr int kKsPitch = 128 + 16;  // LDS row pitch of the transpose column (the pad spreads banks)

struct KsArgs {
    const void* x; int64_t ldx;      // INT8 / E4M3 codes, or bf16 activations (elements)
    const float* xs; int xs_step;    // token scales (INT8, W8A8)
    int M;
    const uint8_t* w; int64_t ldw; int64_t N; int64_t R;
    const float* ws; int ws_step;
    const uint16_t* bias;            // INT8: optional bf16 bias
    void* y; int64_t ldy; int out_kind;  // INT8: out_kind 1 stores the raw int32 sums
    int64_t rbase, rrem;                 // blocks: runs = rbase * G + rrem; bands: rbase = full tiles each
    int npass = 1;                       // passes of T tiles over the workgroup's rows
};

// The workgroup's rows in the chosen LAYOUT: rows(j) is the row of its j-th
// row, or -1 past its range (a run past the last one starts at or beyond N).
template <int LAYOUT>
struct KsRows {
    int64_t G, wg, N, R, rbase, first, count;
    __device__ explicit KsRows(const KsArgs& a)
        : G(gridDim.x), wg(blockIdx.x), N(a.N), R(a.R), rbase(a.rbase) {
        // blocks: the block's first row and its rows (at least one run: G
        // never exceeds the runs)
        first = 4 * (wg * a.rbase + (wg < a.rrem ? wg : a.rrem));
        count = 4 * (a.rbase + (wg < a.rrem ? 1 : 0));
    }
    __device__ int64_t operator()(int64_t j) const {
        if constexpr (LAYOUT == kKsBlocks) {
            const int64_t n = first + j;
            return (j < count && n < N) ? n : -1;
        } else if constexpr (LAYOUT == kKsBands) {
            const int64_t t = j >> 4;
            if (t < rbase) {
                const int64_t n = 16 * (t * G + wg) + (j & 15);
                return n < N ? n : -1;
            }
            const int64_t jj = j - 16 * rbase;
            const int64_t n = 4 * (4 * G * rbase + (jj >> 2) * G + wg) + (jj & 3);
            return n < N ? n : -1;
        } else {
            const int64_t n = 4 * ((j >> 2) * G + wg) + (j & 3);
            return (j < R && n < N) ? n : -1;
        }
    }
    // the row read in place of rows past the range when a whole tile is past it
    __device__ int64_t spare() const { return LAYOUT == kKsBlocks ? first : 4 * wg; }
};

// Load j of tile t (8 rows x 128 bytes per instruction): line j/2 of rows
// 8*(j%2) + lane/8 of the wave's K slice (wb = the slice's first byte plus
// the lane's 16-byte chunk).  Rows past the range read the tile's first row
// instead (the same lines as a lane of the same or the previous load, so no
// extra HBM traffic), or spare() when the whole tile is past the range; they
// are never stored.
template <int L, int LAYOUT>
__device__ __forceinline__ void ks_load_tile(u32x4_t (&buf)[2 * L], const KsRows<LAYOUT>& row, const uint8_t* wb,
                                             int64_t ldw, int t, int lr) {
    const int64_t r0 = row(16 * t), fb = r0 >= 0 ? r0 : row.spare();
    const int64_t ra = row(16 * t + lr), rb = row(16 * t + 8 + lr);
    const uint8_t* p0 = wb + (ra >= 0 ? ra : fb) * ldw;
    const uint8_t* p1 = wb + (rb >= 0 ? rb : fb) * ldw;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        buf[2 * j] = ld_stream(p0 + 128 * j);
        buf[2 * j + 1] = ld_stream(p1 + 128 * j);
    }
}

// XS (one-byte activation codes: INT8, FP8 W8A8): the wave's activation
// slice goes to LDS first, by buffer loads with the LDS bit that each cover
// one 128-byte line of 8 token rows (instead of 16 rows x 64 bytes per
// register load), the weight tiles' loads queue behind it, and the B
// operands are read back from LDS (M = 16, INT8: 18.6 -> 17.7 us).
// LAYOUT: kKsTurn keeps no workgroup more than one run above another and
// streams one band of rows per tile step; kKsBlocks (workgroup b's rows are
// 4*P_b, 4*P_b + 1, ... with P_b = b*rbase + min(b, rrem)) and kKsBands
// (tile t < rbase of workgroup b is rows 16*(t*G + b) .. +15) make a tile's
// outputs 16 adjacent rows, with the same balance.
// MP: the workgroup's rows may take more than one pass (a.npass); without it
// the pass loop folds away and the kernel runs exactly one.
template <int KIND, int L, int T, int XF = kFmtE4M3, int WF = kFmtE4M3, bool XS = false, int LAYOUT = kKsTurn,
          bool MP = false>
__global__ __launch_bounds__(64 * kKsWaves) void gemv_ks_kernel(const KsArgs a) {
    constexpr bool I8 = KIND == kKsI8;
    static_assert(!XS || KIND != kKsF8, "activation staging: one-byte codes");
    constexpr int NQ = 2 * L;                  // loads per tile = 64-K steps of the slice
    constexpr int NX = I8 ? NQ : 2 * NQ;       // B operand registers (16 bytes each) of the slice
    // tiles in flight per wave: as many as the registers hold next to the
    // slice (INT8 above 8 lines, the float kinds above 6: one)
    constexpr int DMAX = I8 ? (L <= 6 ? 3 : (L <= 8 ? 2 : 1)) : (L <= 6 ? 2 : 1);
    constexpr int D = T < DMAX ? T : DMAX;
    typedef typename std::conditional<I8, i32x4_t, f32x4_t>::type acc_t;
    __shared__ __align__(16) uint8_t col[kKsWaves][16 * kKsPitch];
    __shared__ acc_t part[T][kKsWaves][64];
    __shared__ __align__(16) uint8_t xst[XS ? kKsWaves : 1][XS ? NQ * 1024 : 16];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int mi = lane & 15, mg = lane >> 4, lr = lane >> 3, lp = lane & 7;
    const KsRows<LAYOUT> row(a);
    const int64_t k0 = (int64_t)wv * (L * 128);
    const uint8_t* wb = a.w + k0 + 16 * lp;
    uint8_t* cp = col[wv];
    auto load_tile = [&](u32x4_t (&buf)[NQ], int t) { ks_load_tile<L, LAYOUT>(buf, row, wb, a.ldw, t, lr); };

    if constexpr (XS) {
        // load 2j + hh: line j of token rows 8hh + lane/8 (token 0 past M),
        // the chunk that belongs in slot lane%8 (chunk c of row r sits at
        // c ^ (r % 8), so the B reads below hit distinct banks)
        const int t0 = lr < a.M ? lr : 0, t1 = 8 + lr < a.M ? 8 + lr : 0;
        const uint32_t ch = 16u * (uint32_t)(lp ^ lr);
        const uint32_t o0 = (uint32_t)(t0 * a.ldx + k0) + ch, o1 = (uint32_t)(t1 * a.ldx + k0) + ch;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)((a.M - 1) * a.ldx + L * 128 * kKsWaves),
                                              0x00020000);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(xst[wv] + (2 * j) * 1024), 16, o0 + 128 * j, 0,
                                                     0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(xst[wv] + (2 * j + 1) * 1024), 16,
                                                     o1 + 128 * j, 0, 0, 0);
        }
    }
    u32x4_t bufs[D][NQ];
    load_tile(bufs[0], 0);
    if constexpr (XS) {  // every tile in flight before the staged slice is read back
#pragma unroll
        for (int d = 1; d < D; ++d) load_tile(bufs[d], d);
    }
    // the wave's K slice of token lane%16 (zero past M): 64-K step s covers
    // K = k0 + 64s + 16*(lane/16) + [0, 16)
    u32x4_t xb[NX];
    {
        const bool xon = mi < a.M;
        const int64_t m = xon ? mi : 0;
        if constexpr (KIND == kKsF8) {
            const uint16_t* xr = (const uint16_t*)a.x + m * a.ldx + k0 + 16 * mg;
#pragma unroll
            for (int h = 0; h < NX; ++h) {  // h = 2s + half
                const u32x4_t v = ld16(xr + 64 * (h >> 1) + 8 * (h & 1));
                xb[h] = xon ? v : u32x4_t{0, 0, 0, 0};
            }
        } else if constexpr (XS) {
            const uint8_t* xr = xst[wv] + (mi >> 3) * 1024 + (mi & 7) * 128;
#pragma unroll
            for (int s = 0; s < NQ; ++s) {  // s = 2j + h: line j, chunk 4h + lane/16
                const u32x4_t v = *(const u32x4_t*)(xr + (s >> 1) * 2048 + 16 * ((4 * (s & 1) + mg) ^ (mi & 7)));
                const u32x4_t c = xon ? v : u32x4_t{0, 0, 0, 0};
                if constexpr (I8) {
                    xb[s] = c;
                } else {
                    bf16x8_t lo, hi;
                    fp8x16_to_bf16x8x2<XF>(c, lo, hi);
                    xb[2 * s] = __builtin_bit_cast(u32x4_t, lo);
                    xb[2 * s + 1] = __builtin_bit_cast(u32x4_t, hi);
                }
            }
        } else {
            const uint8_t* xr = (const uint8_t*)a.x + m * a.ldx + k0 + 16 * mg;
#pragma unroll
            for (int s = 0; s < NQ; ++s) {
                const u32x4_t v = ld16(xr + 64 * s);
                const u32x4_t c = xon ? v : u32x4_t{0, 0, 0, 0};
                if constexpr (I8) {
                    xb[s] = c;
                } else {
                    bf16x8_t lo, hi;
                    fp8x16_to_bf16x8x2<XF>(c, lo, hi);
                    xb[2 * s] = __builtin_bit_cast(u32x4_t, lo);
                    xb[2 * s + 1] = __builtin_bit_cast(u32x4_t, hi);
                }
            }
        }
    }
    if constexpr (!XS) {
#pragma unroll
        for (int d = 1; d < D; ++d) load_tile(bufs[d], d);
    }

    // pass p covers the workgroup's tiles p*T .. p*T + T - 1 (one pass unless
    // a workgroup has more rows than T tiles hold)
    for (int tb = 0;; tb += T) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            u32x4_t (&buf)[NQ] = bufs[t % D];
            acc_t acc = {};
#pragma unroll
            for (int j = 0; j < L; ++j) {
                *(u32x4_t*)(cp + lr * kKsPitch + 16 * lp) = buf[2 * j];
                *(u32x4_t*)(cp + (8 + lr) * kKsPitch + 16 * lp) = buf[2 * j + 1];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int s = 2 * j + h;
                    const u32x4_t wa = *(const u32x4_t*)(cp + mi * kKsPitch + 64 * h + 16 * mg);
                    if constexpr (I8) {
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, wa),
                                                                   __builtin_bit_cast(i32x4_t, xb[s]), acc, 0, 0, 0);
                    } else {
                        bf16x8_t a0, a1;
                        fp8x16_to_bf16x8x2<WF>(wa, a0, a1);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8_t, xb[2 * s]), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, xb[2 * s + 1]), acc, 0, 0, 0);
                    }
                }
            }
            part[t][wv][lane] = acc;
            if (t + D < T) load_tile(buf, tb + t + D);
        }
        __syncthreads();

        for (int t = wv; t < T; t += kKsWaves) {
            acc_t acc = part[t][0][lane];
#pragma unroll
            for (int q = 1; q < kKsWaves; ++q) acc += part[t][q][lane];
            if (mi >= a.M) continue;
            // rows n0 .. n0+3 (one run; blocks are whole runs, so only N can cut it)
            const int64_t n0 = row(16 * (tb + t) + 4 * mg);
            if (n0 < 0) continue;
            const int nv = a.N - n0 < 4 ? (int)(a.N - n0) : 4;
            if constexpr (I8) {
                if (a.out_kind == 1) {
                    int32_t* yp = (int32_t*)a.y + mi * a.ldy + n0;
                    for (int r = 0; r < nv; ++r) yp[r] = acc[r];
                    continue;
                }
            }
            uint16_t o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = n0 + (r < nv ? r : 0);
                if constexpr (I8) {
                    float v = (float)acc[r];
                    v = v * a.xs[mi * a.xs_step];
                    v = v * a.ws[n * a.ws_step];
                    o[r] = f32_to_bf16(v);
                    if (a.bias) o[r] = f32_to_bf16(bf16_to_f32(o[r]) + bf16_to_f32(a.bias[n]));
                } else if constexpr (KIND == kKsW8A8) {
                    float v = acc[r] * a.xs[mi * a.xs_step];
                    v = v * a.ws[n * a.ws_step];
                    o[r] = f32_to_bf16(v);
                } else {
                    o[r] = f32_to_bf16(acc[r] * a.ws[n * a.ws_step]);
                }
            }
            // element-wise stores: one 8-byte store behind a run-time alignment
            // test measured 28-34 us against 16.4-18.4 us for the whole kernel
            uint16_t* yp = (uint16_t*)a.y + mi * a.ldy + n0;
            for (int r = 0; r < nv; ++r) yp[r] = o[r];
        }
        if (!MP || tb + T >= a.npass * T) break;
        __syncthreads();  // every wave has read part[] before the next pass writes it
#pragma unroll
        for (int d = 0; d < D; ++d) load_tile(bufs[d], tb + T + d);
    }
}

}  // namespace qlin
