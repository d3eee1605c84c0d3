// moe.hip -- top-k routed MXFP4 expert GEMV for gfx950 [DSV4 section 9.3;
// element/scale formats of the OCP MX spec: E2M1 elements, one UE8M0 scale
// per 32 consecutive K elements].
//
// Stage 1+2 (moe_expert_kernel, persistent wavefronts):
//   * every wave reads the M*topk routing ids into LDS and lists the live
//     experts in order of first appearance (pairs whose id is out of range
//     are dropped) -- the bucketing is recomputed per wave, so no host sync
//     and no extra launch is needed;
//   * work item = (live expert u, tile of 4 rows); waves stride over the
//     items.  For an item, the pairs routed to the expert are gathered and
//     the expert's rows are streamed once for up to T pairs at a time;
//   * a 16-byte weight chunk is 32 E2M1 codes = exactly one UE8M0 block, so
//     each lane folds its block scale into its chunk partial before the DPP
//     row reduction; fp32 partial rows go to the workspace, one per pair.
// Stage 3 (moe_combine_kernel): y[t,n] = bf16(sum_j g[t,j] * part[t,j,n]) in
// slot order j = 0..topk-1 (deterministic).
#include "qlin_device.hpp"
#include "qlin_launch.hpp"

namespace qlin {

constexpr int kMaxPairs = 256;  // M <= 16, topk <= 16

template <int T>
__global__ __launch_bounds__(64) void moe_expert_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t K,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ s, int64_t E, int64_t N,
    const int32_t* __restrict__ ids, int topk, float* __restrict__ part) {
    __shared__ int32_t sid[kMaxPairs];
    __shared__ int32_t live[kMaxPairs];
    __shared__ int32_t plist[kMaxPairs];
    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int npairs = M * topk;

    for (int p = lane; p < npairs; p += 64) {
        const int32_t e = ids[p];
        sid[p] = (e >= 0 && e < E) ? e : -1;
    }
    __syncthreads();
    // live experts in order of first appearance
    int nlive = 0;
    for (int base = 0; base < npairs; base += 64) {
        const int p = base + lane;
        bool first = false;
        if (p < npairs && sid[p] >= 0) {
            first = true;
            for (int q = 0; q < p; ++q) first = first && (sid[q] != sid[p]);
        }
        const uint64_t mask = __ballot(first);
        const int rank = __popcll(mask & ((1ull << lane) - 1ull));
        if (first) live[nlive + rank] = sid[p];
        nlive += __popcll(mask);
    }
    __syncthreads();

    const int64_t tiles = (N + 3) / 4;
    const int64_t items = (int64_t)nlive * tiles;
    const int64_t kchunks = K >> 5;  // 32 codes (16 bytes) per chunk
    const int64_t wrow_bytes = K >> 1;

    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int u = (int)(it / tiles);
        const int64_t n = (it % tiles) * 4 + g;
        const int64_t nc = n < N ? n : N - 1;
        const int e = live[u];
        // pairs routed to expert e, in pair order
        int cnt = 0;
        for (int base = 0; base < npairs; base += 64) {
            const int p = base + lane;
            const bool hit = p < npairs && sid[p] == e;
            const uint64_t mask = __ballot(hit);
            const int rank = __popcll(mask & ((1ull << lane) - 1ull));
            __syncthreads();
            if (hit) plist[cnt + rank] = p;
            cnt += __popcll(mask);
        }
        __syncthreads();

        const uint8_t* wr = w + ((int64_t)e * N + nc) * wrow_bytes;
        const uint8_t* sr = s + ((int64_t)e * N + nc) * (K >> 5);
        for (int pb = 0; pb < cnt; pb += T) {
            float acc[T];
            const uint16_t* xr[T];
#pragma unroll
            for (int q = 0; q < T; ++q) {
                acc[q] = 0.0f;
                const int pq = pb + q < cnt ? plist[pb + q] : plist[pb];
                xr[q] = x + (int64_t)(pq / topk) * ldx;
            }
            for (int64_t c = j; c < kchunks; c += 16) {
                const u32x4_t wv = ld_stream(wr + c * 16);
                const float sc = ue8m0_to_f32(sr[c]);
                bf16x2_t wb[16];
                e2m1x8_to_bf16(wv.x, wb + 0);
                e2m1x8_to_bf16(wv.y, wb + 4);
                e2m1x8_to_bf16(wv.z, wb + 8);
                e2m1x8_to_bf16(wv.w, wb + 12);
#pragma unroll
                for (int q = 0; q < T; ++q) {
                    if (pb + q < cnt) {  // wave-uniform
                        const uint16_t* xp = xr[q] + c * 32;
                        const u32x4_t x0 = ld16(xp), x1 = ld16(xp + 8), x2 = ld16(xp + 16), x3 = ld16(xp + 24);
                        const uint32_t xv[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
                        float loc = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) loc = dot2(wb[i], as_bf16x2(xv[i]), loc);
                        acc[q] += loc * sc;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < T; ++q) {
                if (pb + q < cnt) {
                    const float v = row_sum_f32(acc[q]);
                    if (j == (q & 15) && n < N) part[(int64_t)plist[pb + q] * N + n] = v;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void moe_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ids, const float* __restrict__ gw,
    int M, int topk, int64_t E, int64_t N, uint16_t* __restrict__ y, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int t = (int)(i / N);
    const int64_t n = i % N;
    float acc = 0.0f;
    for (int jj = 0; jj < topk; ++jj) {
        const int32_t e = ids[t * topk + jj];
        if (e >= 0 && e < E) acc = fmaf(gw[t * topk + jj], part[(int64_t)(t * topk + jj) * N + n], acc);
    }
    y[t * ldy + n] = f32_to_bf16(acc);
}

template <int T>
static hipError_t launch_moe_t(const MoeArgs& a, hipStream_t st) {
    const int64_t npairs = a.M * a.topk;
    const int64_t max_live = npairs < a.E ? npairs : a.E;
    const int64_t items = max_live * ((a.N + 3) / 4);
    const int64_t grid = items < 8192 ? items : 8192;
    hipLaunchKernelGGL((moe_expert_kernel<T>), dim3((unsigned)grid), dim3(64), 0, st,
                       a.x, a.ldx, (int)a.M, a.K, a.w, a.s, a.E, a.N, a.ids, (int)a.topk, a.part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t total = a.M * a.N;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       a.part, a.ids, a.gw, (int)a.M, (int)a.topk, a.E, a.N, a.y, a.ldy);
    return hipGetLastError();
}

hipError_t launch_moe_mxfp4(const MoeArgs& a, hipStream_t st) {
    if (a.M <= 1) return launch_moe_t<1>(a, st);
    if (a.M <= 2) return launch_moe_t<2>(a, st);
    if (a.M <= 4) return launch_moe_t<4>(a, st);
    return launch_moe_t<8>(a, st);
}

}  // namespace qlin
