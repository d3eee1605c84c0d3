// routing.hip -- on-device MoE routing for gfx950: router logits, top-k and
// the routing weights (softmax over the selected logits).  The pages name the
// routing fast path (M = 1, bit-exact, must stay on) without its scoring
// function; the plain reading used here is a bias-free bf16 router, top-k by
// logit with ties to the lower expert id, and softmax over the k selected
// logits [DSV4 sections 0.1/0.2 (routing Q1), 9.3].
#include "gemv_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

constexpr int kRouterMaxM = 16;
constexpr int kTopkMaxE = 1024;  // one thread per expert in the top-k kernel

// logit[m][e] = sum_k x[m][k] * wr[e][k].  One 1024-lane workgroup per
// expert row, so that every lane issues its (at most RV) 16-byte loads of the
// router row and of each token's x at once -- a single memory round trip;
// v_dot2_f32_bf16 into one fp32 partial per token; DPP row sums, then the 16
// waves are added through LDS in wave order (deterministic).
constexpr int kRouterThreads = 1024;
constexpr int kRouterRV = 4;  // 16-byte vectors per lane: H <= 4 * 1024 * 8 = 32768

__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t H,
    const uint16_t* __restrict__ wr, int64_t E, float* __restrict__ logits) {
    constexpr int W = kRouterThreads / 64;
    __shared__ float part[W][kRouterMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t e = blockIdx.x;
    const int64_t nvec = H >> 3;
    u32x4_t wv8[kRouterRV];
#pragma unroll
    for (int r = 0; r < kRouterRV; ++r) {
        const int64_t v = tid + (int64_t)r * kRouterThreads;
        wv8[r] = v < nvec ? ld16(wr + e * H + v * 8) : u32x4_t{0, 0, 0, 0};
    }
    float acc[kRouterMaxM];
#pragma unroll
    for (int m = 0; m < kRouterMaxM; ++m) {
        acc[m] = 0.0f;
        if (m < M) {
#pragma unroll
            for (int r = 0; r < kRouterRV; ++r) {
                const int64_t v = tid + (int64_t)r * kRouterThreads;
                if (v < nvec) {
                    const u32x4_t xv = ld16(x + m * ldx + v * 8);
                    float a = acc[m];
                    a = dot2(as_bf16x2(wv8[r].x), as_bf16x2(xv.x), a);
                    a = dot2(as_bf16x2(wv8[r].y), as_bf16x2(xv.y), a);
                    a = dot2(as_bf16x2(wv8[r].z), as_bf16x2(xv.z), a);
                    a = dot2(as_bf16x2(wv8[r].w), as_bf16x2(xv.w), a);
                    acc[m] = a;
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < kRouterMaxM; ++m)
        if (m < M) {
            const float a = group_sum<64>(acc[m]);
            if (lane == 0) part[wv][m] = a;
        }
    __syncthreads();
    if (tid < M) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < W; ++q) sum += part[q][tid];
        logits[tid * E + e] = sum;
    }
}

// One workgroup per token, one thread per expert (E <= 1024).  The logits go
// to LDS; thread e counts the experts ranked above it (a larger logit, or an
// equal one with a lower id -- a NaN logit counts as -inf), so the ranks are
// a permutation and rank < k selects the top k in order.  The selected
// thread writes its id; the weights are exp(l_r - l_0) / sum over the k
// selected, summed in slot order by one thread (deterministic).
__global__ __launch_bounds__(kTopkMaxE) void topk_softmax_kernel(
    const float* __restrict__ logits, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gw) {
    __shared__ float lg[kTopkMaxE];
    __shared__ float sel[16];
    __shared__ float den;
    const int e = threadIdx.x;
    const int64_t m = blockIdx.x;
    float v = -INFINITY;
    if (e < E) {
        const float l = logits[m * E + e];
        v = l != l ? -INFINITY : l;
        lg[e] = v;
    }
    __syncthreads();
    if (e < E) {
        int rank = 0;
        for (int q = 0; q < E; ++q) {
            const float o = lg[q];
            rank += (o > v || (o == v && q < e)) ? 1 : 0;
        }
        if (rank < k) {
            ids[m * k + rank] = e;
            sel[rank] = v;
        }
    }
    __syncthreads();
    if (e == 0) {
        float sum = 0.0f;
        for (int r = 0; r < k; ++r) sum += expf(sel[r] - sel[0]);
        den = sum;
    }
    __syncthreads();
    if (e < k) gw[m * k + e] = expf(sel[e] - sel[0]) / den;
}

hipError_t launch_router(const uint16_t* x, int64_t ldx, int64_t M, int64_t H, const uint16_t* wr, int64_t E,
                         float* logits, hipStream_t st) {
    hipLaunchKernelGGL(router_kernel, dim3((unsigned)E), dim3(kRouterThreads), 0, st, x, ldx, (int)M, H, wr, E,
                       logits);
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int64_t M, int64_t E, int64_t topk, int32_t* ids, float* gw,
                               hipStream_t st) {
    const unsigned threads = (unsigned)((E + 63) / 64 * 64);
    hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)M), dim3(threads), 0, st, logits, (int)E, (int)topk,
                       ids, gw);
    return hipGetLastError();
}

}  // namespace qlin
