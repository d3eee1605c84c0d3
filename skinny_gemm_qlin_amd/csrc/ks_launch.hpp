// ks_launch.hpp -- the plan and the launch of the K-slice decode kernels
// (ks_kernels.hpp).  gemv.hip plans (ks_plan) and picks the kind; the
// launchers below are defined one kind per translation unit (ks_i8.hip,
// ks_f8.hip, ks_w8a8_e4m3.hip, ks_w8a8_e5m2.hip), so that their many tile
// and slice instantiations compile in parallel.
#pragma once
#include <algorithm>

#include "ks_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

struct KsPlan { int L, T; unsigned G; int64_t R; int npass; };

hipError_t launch_ks_i8(const KsArgs& a, const KsPlan& p, hipStream_t st);
hipError_t launch_ks_f8(const KsArgs& a, const KsPlan& p, hipStream_t st);
// FP8 W8A8, E4M3 or E5M2 activation codes; w_fmt: the weights' format
hipError_t launch_ks_w8a8_e4m3(const KsArgs& a, const KsPlan& p, int w_fmt, hipStream_t st);
hipError_t launch_ks_w8a8_e5m2(const KsArgs& a, const KsPlan& p, int w_fmt, hipStream_t st);

template <int KIND, int L, int XF, int WF, bool XS = false, int LAYOUT = kKsTurn>
hipError_t run_ks_t(const KsArgs& a, const KsPlan& p, hipStream_t st) {
    const dim3 grid(p.G), block(64 * kKsWaves);
    if (p.npass > 1) {  // then 4 <= T <= kKsMaxTiles
        switch (p.T) {
            case 4: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 4, XF, WF, XS, LAYOUT, true>), grid, block, 0, st, a); break;
            case 5: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 5, XF, WF, XS, LAYOUT, true>), grid, block, 0, st, a); break;
            default: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 6, XF, WF, XS, LAYOUT, true>), grid, block, 0, st, a); break;
        }
        return hipGetLastError();
    }
    switch (p.T) {
        case 1: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 1, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 2, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 3, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 4, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
        case 5: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 5, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((gemv_ks_kernel<KIND, L, 6, XF, WF, XS, LAYOUT>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

// One-byte activation codes (INT8, FP8 W8A8) from kKsStageXMinM tokens,
// with at most 5 lines per slice (LDS: the staged slices take 16 KB x L
// next to the transpose columns and the partial tiles) and the activation
// block addressable with 32-bit offsets: the slice is staged through LDS
// (XS; INT8 M = 4 / 8 / 16: 16.5 / 17.0 / 18.6 -> 16.4 / 16.8 / 17.7 us).
constexpr int64_t kKsStageXMinM = 4;
inline bool ks_stage_x(const KsArgs& a, const KsPlan& p) {
    return a.M >= kKsStageXMinM && p.L <= 5 && (int64_t)(a.M - 1) * a.ldx + 1024 * p.L <= INT32_MAX;
}

// Row layout per kind and token count (17408 x 5120, GEMV alone, against
// the runs dealt out in turn): INT8 with contiguous blocks +0.5 / +0.15 /
// -0.3 / -0.5 us at M = 4 / 8 / 12 / 16 (with bands -0.0..-0.3 from 12 but
// +0.5 at 4); FP8 W8A8 with bands ~0 / -0.4 / -0.4 / -0.7 us; E4M3
// weight-only with bands ~0 / ~0 / -0.4 / -0.7 us (with blocks +0.5 to +0.7
// at every M).
inline int ks_layout(int kind, int64_t M) {
    if (kind == kKsI8) return M >= 12 ? kKsBlocks : kKsTurn;
    if (kind == kKsW8A8) return M >= 8 ? kKsBands : kKsTurn;
    return M >= 12 ? kKsBands : kKsTurn;
}

template <int KIND, int XF, int WF, bool XS, int LAYOUT>
hipError_t run_ks_l(const KsArgs& a, const KsPlan& p, hipStream_t st) {
    switch (p.L) {
        case 2: return run_ks_t<KIND, 2, XF, WF, XS, LAYOUT>(a, p, st);
        case 3: return run_ks_t<KIND, 3, XF, WF, XS, LAYOUT>(a, p, st);
        case 4: return run_ks_t<KIND, 4, XF, WF, XS, LAYOUT>(a, p, st);
        default: return run_ks_t<KIND, 5, XF, WF, XS, LAYOUT>(a, p, st);  // L <= 5 on these paths
    }
}

template <int KIND, int XF = kFmtE4M3, int WF = kFmtE4M3>
hipError_t run_ks(const KsArgs& a, const KsPlan& p, hipStream_t st) {
    const int layout = ks_layout(KIND, a.M);
    KsArgs b = a;
    b.npass = p.npass;
    const int64_t runs = (a.N + 3) / 4;
    if (layout == kKsBlocks) {
        b.rbase = runs / p.G;
        b.rrem = runs - b.rbase * p.G;
    } else if (layout == kKsBands) {
        b.rbase = runs / (4 * (int64_t)p.G);
        b.rrem = 0;
    }
    if constexpr (KIND != kKsF8) {
        if (ks_stage_x(a, p)) {
            if constexpr (KIND == kKsI8) {
                if (layout == kKsBlocks) return run_ks_l<KIND, XF, WF, true, kKsBlocks>(b, p, st);
            } else {
                if (layout == kKsBands) return run_ks_l<KIND, XF, WF, true, kKsBands>(b, p, st);
            }
            return run_ks_l<KIND, XF, WF, true, kKsTurn>(b, p, st);
        }
    } else {
        if (layout == kKsBands && p.L <= 5) return run_ks_l<KIND, XF, WF, false, kKsBands>(b, p, st);
    }
    switch (p.L) {
        case 2: return run_ks_t<KIND, 2, XF, WF>(b, p, st);
        case 3: return run_ks_t<KIND, 3, XF, WF>(b, p, st);
        case 4: return run_ks_t<KIND, 4, XF, WF>(b, p, st);
        case 5: return run_ks_t<KIND, 5, XF, WF>(b, p, st);
        case 6: return run_ks_t<KIND, 6, XF, WF>(b, p, st);
        case 7: return run_ks_t<KIND, 7, XF, WF>(b, p, st);
        case 8: return run_ks_t<KIND, 8, XF, WF>(b, p, st);
        default:
            if constexpr (KIND == kKsI8) {
                switch (p.L) {
                    case 9: return run_ks_t<KIND, 9, XF, WF>(b, p, st);
                    case 10: return run_ks_t<KIND, 10, XF, WF>(b, p, st);
                    case 11: return run_ks_t<KIND, 11, XF, WF>(b, p, st);
                    case 12: return run_ks_t<KIND, 12, XF, WF>(b, p, st);
                    case 13: return run_ks_t<KIND, 13, XF, WF>(b, p, st);
                    default: return run_ks_t<KIND, 14, XF, WF>(b, p, st);
                }
            }
            return hipErrorInvalidValue;  // not reached: ks_plan caps L per kind
    }
}

}  // namespace qlin
