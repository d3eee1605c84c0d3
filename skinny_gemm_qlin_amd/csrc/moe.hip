// moe.hip -- top-k routed MXFP4 expert kernels for gfx950 [DSV4 section 9.3;
// element/scale formats of the OCP MX spec: E2M1 elements, one UE8M0 scale
// per 32 consecutive K elements; SwiGLU of sections 6.6 and 9.4].
//
// moe_expert_kernel: grid = (row tiles) x (expert slots); three modes share it.
//   * bucketing, in every workgroup (no host synchronisation, no extra
//     launch): thread p holds routing pair p (ids outside [0, E) dropped); the
//     first pair of each expert is found with an LDS atomicMin table indexed
//     by expert id (a v_readlane scan when E exceeds the table), live experts
//     are ranked in order of first appearance, slot blockIdx.y takes the
//     expert of that rank and a workgroup past the live count exits at once;
//   * the pairs routed to the expert are listed in pair order and processed
//     T at a time: their activation rows are staged in LDS once per
//     workgroup, then each wave streams 16 weight rows (4 lane groups of 16
//     lanes x 4 rows) with 128-bit loads, U steps of 256 bytes per row in
//     flight, so the expert's weights are read from HBM once per T rows;
//   * a 16-byte chunk is 32 E2M1 codes = exactly one UE8M0 block; a lane
//     widens its codes to bf16 (v_cvt_scalef32_pk_bf16_fp4, exact), dots them
//     with the activations (v_dot2_f32_bf16, fp32) and folds the block scale
//     into its own partial; DPP row reduction.
//   Modes: plain (token rows in, fp32 partial row per pair out); gate/up (a
//   group's 4 rows are 2 gate rows and the 2 matching up rows, and the
//   epilogue writes the bf16 SwiGLU activation per pair); down (the staged
//   rows are the pairs' activation rows, fp32 partial out).
// moe_combine_kernel: y[t,n] = bf16(sum_j g[t,j] * part[t,j,n]) in slot order
// j = 0..topk-1 (deterministic).
#include "gemv_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

constexpr int kMaxPairs = 256;    // M <= 16, topk <= 16
constexpr int kMoeRows = 64;      // rows per workgroup: 4 waves x 4 groups x 4 rows
constexpr int kMoeR = 4;          // rows per 16-lane group
constexpr int64_t kMoeLdsBytes = 64 * 1024;  // activation staging budget per workgroup
constexpr int kMoeTable = 1024;   // experts covered by the first-occurrence table

// Staged activation row layout in LDS: 16 bytes of padding after every 128
// elements, so the 16 lanes of a group (64-byte stride) hit distinct banks.
__host__ __device__ constexpr int64_t moe_pitch(int64_t K) { return K + ((K + 127) >> 7) * 8; }

enum MoeMode { kMoePlain = 0, kMoeGateUp = 1, kMoeDown = 2 };

struct MoeKParams {
    const uint16_t* x;   // staged rows: x[token] (plain, gate/up) or act[pair] (down)
    int64_t ldx;
    int M;
    int64_t K;
    const uint8_t* w;    // E2M1 codes [E][rows][K/2]; rows = N, or 2N (gate rows then up rows)
    const uint8_t* s;    // UE8M0 [E][rows][K/32]
    int64_t E;
    int64_t N;           // output rows per expert
    const int32_t* ids;  // [M][topk]
    int topk;
    float* part;         // plain / down: fp32 [M*topk][N]
    uint16_t* act;       // gate/up: bf16 [M*topk][N]
    float alpha, limit;  // gate/up: SwiGLU parameters
};

// silu(alpha * min(gate, limit)) * clamp(up, -limit, limit) [DSV4 sections
// 6.6 and 9.4]; silu(z) = z / (1 + e^-z).
__device__ __forceinline__ float swiglu(float gate, float up, float alpha, float limit) {
    const float gc = gate > limit ? limit : gate;
    const float uc = up > limit ? limit : (up < -limit ? -limit : up);
    const float z = alpha * gc;
    return z / (1.0f + expf(-z)) * uc;
}

template <int MODE>
__host__ __device__ constexpr int moe_rows_per_wg() { return MODE == kMoeGateUp ? kMoeRows / 2 : kMoeRows; }

template <int T, int U, bool TABLE, int MODE>
__global__ __launch_bounds__(256) void moe_expert_kernel(const MoeKParams a) {
    const uint16_t* __restrict__ x = a.x;
    const int64_t ldx = a.ldx, K = a.K, E = a.E, N = a.N;
    const int M = a.M, topk = a.topk;
    const uint8_t* __restrict__ w = a.w;
    const uint8_t* __restrict__ s = a.s;
    const int32_t* __restrict__ ids = a.ids;
    extern __shared__ __align__(16) uint16_t xl[];  // [T][pitch] activation rows of the current pairs
    __shared__ int32_t plist[kMaxPairs];
    __shared__ int32_t firstpos[TABLE ? kMoeTable : 1];
    __shared__ int32_t wcnt[4], hcnt[4];
    __shared__ int32_t sh_e;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int npairs = M * topk;  // <= 256: thread p owns pair p
    const uint64_t below = (1ull << lane) - 1ull;

    int mine = -1;
    if (tid < npairs) {
        const int32_t id = ids[tid];
        mine = (id >= 0 && id < E) ? id : -1;
    }
    if (TABLE)
        for (int i = tid; i < E; i += 256) firstpos[i] = 0x7fffffff;
    if (tid == 0) sh_e = -1;
    bool first;
    if (TABLE) {
        __syncthreads();
        if (mine >= 0) atomicMin(&firstpos[mine], tid);
        __syncthreads();
        first = mine >= 0 && firstpos[mine] == tid;
    } else {
        // first appearance without a table: compare with every earlier pair,
        // its id read back with v_readlane (wave w scans waves 0..w)
        __shared__ int32_t sid[kMaxPairs];
        sid[tid] = mine;
        __syncthreads();
        first = mine >= 0;
        for (int q0 = 0; q0 <= wv * 64; q0 += 64) {
            const int other = sid[q0 + lane];
            const int lim = npairs - q0 < 64 ? npairs - q0 : 64;
            for (int l = 0; l < lim; ++l) {
                const int v = __builtin_amdgcn_readlane(other, l);
                first = first && !(q0 + l < tid && v == mine);
            }
        }
    }
    const uint64_t fm = __ballot(first);
    if (lane == 0) wcnt[wv] = __popcll(fm);
    __syncthreads();
    int base = 0;
    for (int q = 0; q < wv; ++q) base += wcnt[q];
    if (first && base + __popcll(fm & below) == (int)blockIdx.y) sh_e = mine;
    __syncthreads();
    const int e = sh_e;
    if (e < 0) return;  // slot past the number of live experts (workgroup-uniform)
    const bool h = mine == e;
    const uint64_t hm = __ballot(h);
    if (lane == 0) hcnt[wv] = __popcll(hm);
    __syncthreads();
    int hb = 0, cnt = 0;
    for (int q = 0; q < 4; ++q) {
        hb += q < wv ? hcnt[q] : 0;
        cnt += hcnt[q];
    }
    if (h) plist[hb + __popcll(hm & below)] = tid;  // read after the barrier that opens each pass

    const int kchunks = (int)(K >> 5);  // 16-byte chunks (32 codes) per row
    const int nsteps = (kchunks + 15) >> 4;
    const int pitch = (int)moe_pitch(K);
    // output rows of this lane group: 4 (plain, down) or 2 (gate/up: rows r
    // and r + 2 of the group are the gate and up rows of the same output)
    constexpr int kOut = MODE == kMoeGateUp ? kMoeR / 2 : kMoeR;
    const int64_t n0 = (int64_t)blockIdx.x * moe_rows_per_wg<MODE>() + (wv * 4 + g) * kOut;
    const int64_t rows_per_expert = MODE == kMoeGateUp ? 2 * N : N;
    const uint8_t* wr[kMoeR];
    const uint8_t* sr[kMoeR];
#pragma unroll
    for (int r = 0; r < kMoeR; ++r) {
        const int64_t n = n0 + (r % kOut) < N ? n0 + (r % kOut) : N - 1;
        const int64_t row = (MODE == kMoeGateUp && r >= kOut) ? N + n : n;
        wr[r] = w + ((int64_t)e * rows_per_expert + row) * (K >> 1);
        sr[r] = s + ((int64_t)e * rows_per_expert + row) * kchunks;
    }

    for (int pb = 0; pb < cnt; pb += T) {
        const int nt = cnt - pb < T ? cnt - pb : T;
        // stage the activation rows of pairs pb..pb+nt-1, 16 bytes per lane
        __syncthreads();  // the previous pass is done reading xl
        const int vec_per_row = (int)(K >> 3);
        for (int i = tid; i < nt * vec_per_row; i += 256) {
            const int t = i / vec_per_row;
            const int v = i - t * vec_per_row;
            const int64_t row = MODE == kMoeDown ? plist[pb + t] : plist[pb + t] / topk;
            *(u32x4_t*)(xl + t * pitch + v * 8 + (v >> 4) * 8) = ld16(x + row * ldx + (int64_t)v * 8);
        }
        __syncthreads();

        float acc[kMoeR][T];
#pragma unroll
        for (int r = 0; r < kMoeR; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[r][t] = 0.0f;

        for (int st = 0; st < nsteps; st += U) {
            u32x4_t wv_[U][kMoeR];
            uint32_t sb[U][kMoeR];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (st + u < nsteps) {  // wave-uniform
                    const int c = (st + u) * 16 + j;
                    const int cc = c < kchunks ? c : kchunks - 1;
#pragma unroll
                    for (int r = 0; r < kMoeR; ++r) {
                        wv_[u][r] = ld_stream(wr[r] + (int64_t)cc * 16);
                        sb[u][r] = sr[r][cc];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (st + u >= nsteps) break;  // wave-uniform
                const int c = (st + u) * 16 + j;
                const bool ok = c < kchunks;
                const int cc = ok ? c : kchunks - 1;
                // activations of this chunk: 32 bf16 per token from LDS
                u32x4_t xa[T][4];
#pragma unroll
                for (int t = 0; t < T; ++t)
                    if (t < nt) {
                        const uint16_t* xp = xl + t * pitch + cc * 32 + (cc >> 2) * 8;
#pragma unroll
                        for (int q = 0; q < 4; ++q) xa[t][q] = *(const u32x4_t*)(xp + 8 * q);
                    }
#pragma unroll
                for (int r = 0; r < kMoeR; ++r) {
                    bf16x2_t wb[16];
                    e2m1x8_to_bf16(wv_[u][r].x, wb + 0);
                    e2m1x8_to_bf16(wv_[u][r].y, wb + 4);
                    e2m1x8_to_bf16(wv_[u][r].z, wb + 8);
                    e2m1x8_to_bf16(wv_[u][r].w, wb + 12);
                    const float sc = ue8m0_to_f32(sb[u][r]);
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        if (t < nt) {
                            float loc = 0.0f;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                loc = dot2(wb[4 * q + 0], as_bf16x2(xa[t][q].x), loc);
                                loc = dot2(wb[4 * q + 1], as_bf16x2(xa[t][q].y), loc);
                                loc = dot2(wb[4 * q + 2], as_bf16x2(xa[t][q].z), loc);
                                loc = dot2(wb[4 * q + 3], as_bf16x2(xa[t][q].w), loc);
                            }
                            acc[r][t] += ok ? loc * sc : 0.0f;  // a lane past the row end adds 0
                        }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kMoeR; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (t < nt) acc[r][t] = group_sum<16>(acc[r][t]);
#pragma unroll
        for (int r = 0; r < kOut; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (t < nt) {
                    const int64_t n = n0 + r;
                    if (j != ((r * T + t) & 15) || n >= N) continue;
                    const int64_t o = (int64_t)plist[pb + t] * N + n;
                    if (MODE == kMoeGateUp)
                        a.act[o] = f32_to_bf16(swiglu(acc[r][t], acc[r + kOut][t], a.alpha, a.limit));
                    else
                        a.part[o] = acc[r][t];
                }
    }
}

// One thread per output (t, n).  All topk ids, gates and partials are loaded
// before the sum (one memory latency instead of topk); a pair whose id is out
// of range is skipped by a select, so its never-written partial row cannot
// leak into the sum.
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ids, const float* __restrict__ gw,
    int M, int topk, int64_t E, int64_t N, uint16_t* __restrict__ y, int64_t ldy) {
    constexpr int kMaxTopk = 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int t = (int)(i / N);
    const int64_t n = i % N;
    bool ok[kMaxTopk];
    float g[kMaxTopk], v[kMaxTopk];
#pragma unroll
    for (int jj = 0; jj < kMaxTopk; ++jj) {
        ok[jj] = false;
        g[jj] = v[jj] = 0.0f;
        if (jj < topk) {
            const int p = t * topk + jj;
            const int32_t e = ids[p];
            ok[jj] = e >= 0 && e < E;
            g[jj] = gw[p];
            v[jj] = part[(int64_t)p * N + n];
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kMaxTopk; ++jj)
        if (jj < topk) acc = ok[jj] ? fmaf(g[jj], v[jj], acc) : acc;
    y[t * ldy + n] = f32_to_bf16(acc);
}

template <int MODE, int T, bool TABLE>
static hipError_t launch_expert(const MoeKParams& p, hipStream_t st) {
    const int64_t npairs = (int64_t)p.M * p.topk;
    const int64_t slots = npairs < p.E ? npairs : p.E;
    constexpr int rows = moe_rows_per_wg<MODE>();
    dim3 grid((unsigned)((p.N + rows - 1) / rows), (unsigned)slots);
    const size_t lds = (size_t)T * moe_pitch(p.K) * 2;
    hipLaunchKernelGGL((moe_expert_kernel<T, 2, TABLE, MODE>), grid, dim3(256), lds, st, p);
    return hipGetLastError();
}

// Two staged rows per pass (T = 2, U = 2: 122 VGPRs, four waves per SIMD)
// while both fit the LDS budget, else one (K <= 30720 keeps one row within
// it).  Four rows per pass re-read fewer experts but halve the resident
// waves, which costs more than the re-reads at decode batch sizes.
template <int MODE>
static hipError_t launch_expert_any(const MoeKParams& p, hipStream_t st) {
    const bool two = 2 * moe_pitch(p.K) * 2 <= kMoeLdsBytes;
    if (p.E <= kMoeTable) return two ? launch_expert<MODE, 2, true>(p, st) : launch_expert<MODE, 1, true>(p, st);
    return two ? launch_expert<MODE, 2, false>(p, st) : launch_expert<MODE, 1, false>(p, st);
}

static hipError_t launch_combine(const float* part, const int32_t* ids, const float* gw, int64_t M, int64_t topk,
                                 int64_t E, int64_t N, uint16_t* y, int64_t ldy, hipStream_t st) {
    const int64_t total = M * N;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       part, ids, gw, (int)M, (int)topk, E, N, y, ldy);
    return hipGetLastError();
}

hipError_t launch_moe_mxfp4(const MoeArgs& a, hipStream_t st) {
    hipError_t err;
    if (a.M > 16) {  // prefill: sort the pairs by expert, grouped GEMM (moe_prefill.hip)
        int32_t* offs = a.sort;
        int32_t* toffs = offs + a.E + 1;
        int32_t* perm = toffs + a.E + 1;
        err = launch_moe_prefill_mxfp4(a, offs, toffs, perm, st);
        if (err != hipSuccess) return err;
        return launch_combine(a.part, a.ids, a.gw, a.M, a.topk, a.E, a.N, a.y, a.ldy, st);
    }
    MoeKParams p{a.x, a.ldx, (int)a.M, a.K, a.w, a.s, a.E, a.N, a.ids, (int)a.topk, a.part, nullptr, 0.f, 0.f};
    err = launch_expert_any<kMoePlain>(p, st);
    if (err != hipSuccess) return err;
    return launch_combine(a.part, a.ids, a.gw, a.M, a.topk, a.E, a.N, a.y, a.ldy, st);
}

hipError_t launch_moe_ffn_mxfp4(const MoeFfnArgs& a, hipStream_t st) {
    hipError_t err = launch_router(a.x, a.ldx, a.M, a.H, a.wr, a.E, a.logits, st);
    if (err != hipSuccess) return err;
    err = launch_topk_softmax(a.logits, a.M, a.E, a.topk, a.ids, a.gw, st);
    if (err != hipSuccess) return err;
    MoeKParams gu{a.x, a.ldx, (int)a.M, a.H, a.w13, a.s13, a.E, a.I, a.ids, (int)a.topk, nullptr, a.act,
                  a.alpha, a.limit};
    err = launch_expert_any<kMoeGateUp>(gu, st);
    if (err != hipSuccess) return err;
    MoeKParams dn{a.act, a.I, (int)a.M, a.I, a.w2, a.s2, a.E, a.H, a.ids, (int)a.topk, a.part, nullptr, 0.f, 0.f};
    err = launch_expert_any<kMoeDown>(dn, st);
    if (err != hipSuccess) return err;
    return launch_combine(a.part, a.ids, a.gw, a.M, a.topk, a.E, a.H, a.y, a.ldy, st);
}

}  // namespace qlin
