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
constexpr int kTopkMaxE = 1024;  // 16 expert logits per lane

// logit[m][e] = sum_k x[m][k] * wr[e][k].  One 256-lane workgroup per expert
// row: each lane takes 8 K at a time (one 16-byte load of the router row and
// one per token), v_dot2_f32_bf16 into one fp32 partial per token; DPP row
// sums, then across the 4 waves through LDS in wave order (deterministic).
__global__ __launch_bounds__(256) void router_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int M, int64_t H,
    const uint16_t* __restrict__ wr, int64_t E, float* __restrict__ logits) {
    __shared__ float part[4][kRouterMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t e = blockIdx.x;
    const int64_t nvec = H >> 3;
    float acc[kRouterMaxM];
#pragma unroll
    for (int m = 0; m < kRouterMaxM; ++m) acc[m] = 0.0f;
    for (int64_t v = tid; v < nvec; v += 256) {
        const u32x4_t wv8 = ld16(wr + e * H + v * 8);
#pragma unroll
        for (int m = 0; m < kRouterMaxM; ++m)
            if (m < M) {
                const u32x4_t xv = ld16(x + m * ldx + v * 8);
                float a = acc[m];
                a = dot2(as_bf16x2(wv8.x), as_bf16x2(xv.x), a);
                a = dot2(as_bf16x2(wv8.y), as_bf16x2(xv.y), a);
                a = dot2(as_bf16x2(wv8.z), as_bf16x2(xv.z), a);
                a = dot2(as_bf16x2(wv8.w), as_bf16x2(xv.w), a);
                acc[m] = a;
            }
    }
#pragma unroll
    for (int m = 0; m < kRouterMaxM; ++m)
        if (m < M) {
            float a = group_sum<64>(acc[m]);
            if (lane == 0) part[wv][m] = a;
        }
    __syncthreads();
    if (tid < M) logits[tid * E + e] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
}

// One wave per token.  Lane l owns the logits of experts l, l + 64, ...;
// k rounds of a wave argmax (largest logit, ties to the lower expert id; a
// NaN logit is never selected) pick the experts in order; lane j keeps the
// j-th selected logit, and the weights are exp(l_j - l_0) / sum over the k
// selected (l_0 is the largest).
__global__ __launch_bounds__(64) void topk_softmax_kernel(
    const float* __restrict__ logits, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gw) {
    constexpr int Q = kTopkMaxE / 64;
    const int lane = threadIdx.x;
    const int64_t m = blockIdx.x;
    float v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        v[q] = e < E ? logits[m * E + e] : 0.0f;
    }
    uint32_t taken = 0;
    float selv = 0.0f;
    for (int jj = 0; jj < k; ++jj) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = lane + 64 * q;
            if (e < E && !((taken >> q) & 1u) && (v[q] > bv || (v[q] == bv && e < be))) {
                bv = v[q];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if (be != 0x7fffffff && lane == (be & 63)) taken |= 1u << (be >> 6);
        if (lane == jj) selv = bv;
        if (lane == 0) ids[m * k + jj] = be;
    }
    const float mx = __shfl(selv, 0);
    const float ex = lane < k ? expf(selv - mx) : 0.0f;
    float den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (lane < k) gw[m * k + lane] = ex / den;
}

hipError_t launch_router(const uint16_t* x, int64_t ldx, int64_t M, int64_t H, const uint16_t* wr, int64_t E,
                         float* logits, hipStream_t st) {
    hipLaunchKernelGGL(router_kernel, dim3((unsigned)E), dim3(256), 0, st, x, ldx, (int)M, H, wr, E, logits);
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int64_t M, int64_t E, int64_t topk, int32_t* ids, float* gw,
                               hipStream_t st) {
    hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E, (int)topk, ids,
                       gw);
    return hipGetLastError();
}

}  // namespace qlin
