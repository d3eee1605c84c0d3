// moe_prefill.hip -- the MXFP4 expert GEMV behind top-k routing for
// prefill-sized M (> 16 tokens) as a grouped GEMM [DSV4 section 9.3;
// E2M1 elements with one UE8M0 scale per 32 K elements, OCP MX formats].
//
//   moe_sort_kernel   one workgroup: counts the (token, slot) pairs of each
//                     expert, prefix sums of pairs and of pair tiles, and
//                     places every pair into its expert's segment of perm[]
//                     (LDS atomics: the order inside a segment is arbitrary,
//                     which no result depends on -- every pair's row is
//                     computed on its own and the combine sums in slot order);
//   moe_gemm_kernel   grid = (128-row weight tiles) x (upper bound on the
//                     pair tiles); a workgroup finds its expert by binary
//                     search in the tile prefix sums and computes 64 pairs x
//                     128 rows of part[pair][n]: weight codes and scale bytes
//                     and the gathered activation rows go through LDS
//                     (double-buffered, K tiles of 128), the E2M1 codes are
//                     widened by v_cvt_scalef32_pk_bf16_fp4 with the block
//                     scale 2^(s-127) applied in the convert, and multiplied
//                     on the bf16 matrix core (fp32 accumulation);
//   the slot-order combine of moe.hip finishes y.
// All on the device, no host synchronisation.
#include "gemm_kernels.hpp"
#include "qlin_launch.hpp"

namespace qlin {

constexpr int kPfBM = 64;    // pairs per tile
constexpr int kPfTN = 4;     // 16-row MFMA tiles per wave along n
constexpr int kPfBN = 32 * kPfTN;  // weight rows per tile (2 waves along n)
constexpr int kPfBK = 128;   // K per LDS tile
constexpr int kPfWP = kPfBK / 2 + 16;   // LDS pitch of a code row (bytes)
constexpr int kPfXP = kPfBK * 2 + 16;   // LDS pitch of an activation row (bytes)
constexpr int kSortMaxE = 1024;

__global__ __launch_bounds__(1024) void moe_sort_kernel(const int32_t* __restrict__ ids, int P, int E, int bm,
                                                        int32_t* __restrict__ offs, int32_t* __restrict__ toffs,
                                                        int32_t* __restrict__ perm) {
    __shared__ int32_t cnt[kSortMaxE];
    __shared__ int32_t cur[kSortMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int o = 0, to = 0;
        for (int e = 0; e < E; ++e) {
            offs[e] = o;
            toffs[e] = to;
            cur[e] = o;
            o += cnt[e];
            to += (cnt[e] + bm - 1) / bm;
        }
        offs[E] = o;
        toffs[E] = to;
    }
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) perm[atomicAdd(&cur[e], 1)] = p;
    }
}

struct MoeGemmParams {
    const uint16_t* x; int64_t ldx; int64_t K;
    const uint8_t* w; const uint8_t* s; int E; int64_t N; int topk;
    const int32_t* offs; const int32_t* toffs; const int32_t* perm;
    float* part;
};

// 8 E2M1 codes (one dword) -> bf16x8 scaled by sc (exact while the scaled
// values stay in bf16's normal range).
__device__ __forceinline__ bf16x8_t e2m1x8_scaled(uint32_t d, float sc) {
    const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0);
    const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1);
    const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2);
    const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3);
    return bf16x8_t{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
}

// Waves 2 x 2, each kPfTN x 2 MFMA tiles of 16 x 16 (16*kPfTN weight rows x
// 32 pairs).  Activation rows past the tile's pair count are not loaded
// (their output columns are never stored).
// MFMA k-step ks covers K 32*ks .. +31 of the tile (lane group g: 8g .. 8g+7),
// one scale block per weight row.
__global__ __launch_bounds__(256) void moe_gemm_kernel(const MoeGemmParams p) {
    __shared__ __align__(16) uint8_t wt[2][kPfBN * kPfWP];
    __shared__ __align__(16) uint8_t st[2][kPfBN * 4];
    __shared__ __align__(16) uint8_t xt[2][kPfBM * kPfXP];
    __shared__ int32_t prow[kPfBM];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn = wv & 1, wm = wv >> 1, li = lane & 15, lg = lane >> 4;
    const int E = p.E;
    const int64_t K = p.K, N = p.N;

    const int ty = blockIdx.y;
    if (ty >= p.toffs[E]) return;  // workgroup-uniform: past the tiles the routing produced
    int lo = 0, hi = E;             // largest e with toffs[e] <= ty (then ty < toffs[e + 1])
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.toffs[mid] <= ty) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int base = p.offs[e] + (ty - p.toffs[e]) * kPfBM;
    const int cnt = min(kPfBM, p.offs[e + 1] - base);
    if (tid < kPfBM) prow[tid] = p.perm[base + (tid < cnt ? tid : 0)];
    __syncthreads();

    const int64_t n0 = (int64_t)blockIdx.x * kPfBN;
    const int64_t kcode = K >> 1, ksc = K >> 5;
    // weight codes: chunk c -> (row c/4, 16-byte column c%4); scales: (row c/4, byte c%4)
    constexpr int WCH = kPfBN * 4 / 256;
    const uint8_t* wsrc[WCH];
    const uint8_t* ssrc[WCH];
    int wrow[WCH];
    const int wc = tid & 3;
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        wrow[i] = (tid + 256 * i) >> 2;
        const int64_t n = n0 + wrow[i] < N ? n0 + wrow[i] : N - 1;
        wsrc[i] = p.w + ((int64_t)e * N + n) * kcode + wc * 16;
        ssrc[i] = p.s + ((int64_t)e * N + n) * ksc + wc;
    }
    // activations: 4 chunks per lane, chunk c -> (pair row c/16, 16-byte column c%16)
    const uint16_t* xsrc[4];
    int xdst[4], xcol[4];
    bool xlive[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256, r = c >> 4;
        xcol[i] = (c & 15) * 8;  // element offset
        xlive[i] = r < cnt;
        xsrc[i] = p.x + (int64_t)(prow[r] / p.topk) * p.ldx + xcol[i];
        xdst[i] = r * kPfXP + (c & 15) * 16;
    }
    const int64_t ktiles = (K + kPfBK - 1) / kPfBK;
    // a ring of three register sets: the loads of K tiles kt+1 .. kt+3 are
    // in flight while tile kt is multiplied (one tile in flight is not enough
    // to cover the memory latency with two workgroups per CU)
    struct Stage {
        u32x4_t w[WCH], x[4];
        uint32_t s[WCH];
    };
    Stage rs0, rs1, rs2;
    // loads are unconditional (addresses clamped into the row, values past K
    // or of dead pair rows replaced by zeros) so that no exec-mask branch
    // forces the loads of the ring to drain
    auto gload = [&](Stage& r, int64_t kt) {
        const int64_t ktc = kt < ktiles ? kt : ktiles - 1;
        const int64_t kc = ktc * kPfBK;
        const bool kin = kc + wc * 32 < K;
        const int64_t wo = kin ? ktc * (kPfBK / 2) : 0, so = kin ? ktc * 4 : 0;
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const u32x4_t v = ld_stream(wsrc[i] + wo);
            const uint32_t sb = ssrc[i][so];
            r.w[i] = kin ? v : u32x4_t{0, 0, 0, 0};
            r.s[i] = kin ? sb : 127u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = xlive[i] && kc + xcol[i] < K;
            const u32x4_t v = ld16(xsrc[i] + (ok ? kc : 0));
            r.x[i] = ok ? v : u32x4_t{0, 0, 0, 0};
        }
    };
    auto lstore = [&](const Stage& r, int b) {
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            *(u32x4_t*)(wt[b] + wrow[i] * kPfWP + wc * 16) = r.w[i];
            st[b][wrow[i] * 4 + wc] = (uint8_t)r.s[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4_t*)(xt[b] + xdst[i]) = r.x[i];
    };

    f32x4_t acc[kPfTN][2];
#pragma unroll
    for (int i = 0; i < kPfTN; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // step kt: refill the free set with tile kt+3, multiply LDS buffer kt&1,
    // store tile kt+1 from its set into the other buffer, barrier
    auto step = [&](int64_t kt, Stage& freed, const Stage& next) {
        const int b = (int)(kt & 1);
        gload(freed, kt + 3);
#pragma unroll
        for (int ks = 0; ks < kPfBK / 32; ++ks) {
            bf16x8_t a[kPfTN], bb[2];
#pragma unroll
            for (int i = 0; i < kPfTN; ++i) {
                const int r = wn * 16 * kPfTN + i * 16 + li;
                const uint32_t codes = *(const uint32_t*)(wt[b] + r * kPfWP + ks * 16 + lg * 4);
                a[i] = e2m1x8_scaled(codes, ue8m0_to_f32(st[b][r * 4 + ks]));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bb[j] = *(const bf16x8_t*)(xt[b] + (wm * 32 + j * 16 + li) * kPfXP + ks * 64 + lg * 16);
#pragma unroll
            for (int i = 0; i < kPfTN; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < ktiles) lstore(next, b ^ 1);
        __syncthreads();
    };
    gload(rs0, 0);
    gload(rs1, 1);
    gload(rs2, 2);
    lstore(rs0, 0);
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; kt += 3) {
        step(kt, rs0, rs1);
        if (kt + 1 < ktiles) step(kt + 1, rs1, rs2);
        if (kt + 2 < ktiles) step(kt + 2, rs2, rs0);
    }

    // lane holds D[n = 4*lg + r][pair = li] of each 16 x 16 tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int tr = wm * 32 + j * 16 + li;
        if (tr >= cnt) continue;
        float* prow_out = p.part + (int64_t)prow[tr] * N;
#pragma unroll
        for (int i = 0; i < kPfTN; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t n = n0 + wn * 16 * kPfTN + i * 16 + 4 * lg + r;
                if (n < N) prow_out[n] = acc[i][j][r];
            }
    }
}

// ------------------------------------------------------------------ direct-to-LDS variant (K % 256 == 0)
// Grid and expert lookup as moe_gemm_kernel, 32 pairs x 128 weight rows per
// workgroup, K tiles of 256 in a two-stage LDS ring filled by
// global_load_lds (as gemm_dma_kernel): a weight row's codes are one whole
// 128-byte line per tile (16-byte chunk c at c ^ ((row >> 1) & 7)), its 8
// scale bytes come with 4-byte loads, and the live pairs' activation rows
// are gathered 512 bytes per row (chunk c at c ^ (row & 15); dead rows are
// not loaded).  Wave w owns weight rows 32w .. 32w+31 against all 32 pairs:
// per 32 K one scale byte per row, applied in the E2M1 -> bf16 convert,
// and two v_mfma_f32_32x32x16_bf16 (a lane's 16 K: codes 0-7, then 8-15).
constexpr int kPdBN = 128, kPdBK = 256;

template <int BM>  // pairs per tile (a multiple of 32)
__global__ __launch_bounds__(256) void moe_gemm_dma_kernel(const MoeGemmParams p) {
    constexpr int TM = BM / 32;             // 32 x 32 tiles per wave along the pairs
    constexpr int XI = BM / 8;              // activation load instructions per wave (2 rows each)
    constexpr int WT = kPdBN * kPdBK / 2;   // code bytes per stage (128 rows x 128 B)
    constexpr int STB = kPdBN * 8;          // scale bytes per stage (8 per row)
    constexpr int XRB = kPdBK * 2;          // activation row bytes per stage
    constexpr int XT = BM * XRB;
    constexpr int ST = WT + STB + XT;
    __shared__ __align__(16) uint8_t lds[2 * ST];
    __shared__ int32_t prow[BM];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = p.E;
    const int64_t K = p.K, N = p.N;

    const int ty = blockIdx.y;
    if (ty >= p.toffs[E]) return;  // workgroup-uniform: past the tiles the routing produced
    int lo = 0, hi = E;             // largest e with toffs[e] <= ty
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.toffs[mid] <= ty) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int base = p.offs[e] + (ty - p.toffs[e]) * BM;
    const int cnt = min(BM, p.offs[e + 1] - base);
    if (tid < BM) prow[tid] = p.perm[base + (tid < cnt ? tid : 0)];
    __syncthreads();

    const int64_t n0 = (int64_t)blockIdx.x * kPdBN;
    const int64_t kcode = K >> 1, ksc = K >> 5;
    // weight codes: instruction i of wave w covers rows (4w + i)*8 .. +7
    const uint8_t* wsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wv * 4 + i) * 8 + (lane >> 3);
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        wsrc[i] = p.w + ((int64_t)e * N + n) * kcode + (((lane & 7) ^ dma_swz(r)) * 16);
    }
    // scales: wave w covers rows 32w .. 32w+31, two dwords per row
    const uint8_t* ssrc;
    {
        const int r = wv * 32 + (lane >> 1);
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        ssrc = p.s + ((int64_t)e * N + n) * ksc + (lane & 1) * 4;
    }
    // activations: instruction i of wave w covers pair rows (XI*w + i)*2 .. +1
    const uint8_t* xsrc[XI];
    bool xlive[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = (wv * XI + i) * 2 + (lane >> 5);
        xlive[i] = r < cnt;
        xsrc[i] = (const uint8_t*)(p.x + (int64_t)(prow[r] / p.topk) * p.ldx) + (((lane & 31) ^ (r & 15)) * 16);
    }
    auto issue = [&](int64_t kt, int slot) {
        uint8_t* b = lds + slot * ST;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + kt * (kPdBK / 2)),
                                             (lds_void_t*)(b + (wv * 4 + i) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + kt * 8), (lds_void_t*)(b + WT + wv * 256), 4, 0, 0);
#pragma unroll
        for (int i = 0; i < XI; ++i)
            if (xlive[i])  // dead pair rows are never read back
                __builtin_amdgcn_global_load_lds((const void*)(xsrc[i] + kt * XRB),
                                                 (lds_void_t*)(b + WT + STB + (wv * XI + i) * 1024), 16, 0, 0);
    };

    const int row = lane & 31, half = lane >> 5;
    const int ar = wv * 32 + row;  // this lane's weight row in the tile
    // two accumulators per tile (the two 16-K halves of each step) so that a
    // wave has two independent MFMA chains; summed once at the end
    f32x16_t acc[TM][2];
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[j][0] = acc[j][1] = f32x16_t{};
    const int64_t ktiles = K / kPdBK;
    issue(0, 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        wait_vmcnt<0>();
        stage_barrier();
        issue(kt + 1 < ktiles ? kt + 1 : kt, (int)((kt + 1) & 1));  // unconditional (see gemm_dma_kernel)
        const uint8_t* Wt = lds + (kt & 1) * ST;
        const uint8_t* St = Wt + WT;
        const uint8_t* Xt = St + STB;
#pragma unroll
        for (int ks = 0; ks < kPdBK / 32; ++ks) {
            const uint2 codes = *(const uint2*)(Wt + ar * 128 + ((ks ^ dma_swz(ar)) * 16) + half * 8);
            const float sc = ue8m0_to_f32(St[ar * 8 + ks]);
            const bf16x8_t a0 = e2m1x8_scaled(codes.x, sc), a1 = e2m1x8_scaled(codes.y, sc);
            const int c0 = 4 * ks + 2 * half;
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int xr = j * 32 + row;
                const bf16x8_t b0 = *(const bf16x8_t*)(Xt + xr * XRB + ((c0 ^ (xr & 15)) * 16));
                const bf16x8_t b1 = *(const bf16x8_t*)(Xt + xr * XRB + (((c0 + 1) ^ (xr & 15)) * 16));
                acc[j][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[j][0], 0, 0, 0);
                acc[j][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[j][1], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();  // no load into LDS outlives the workgroup

    // register r: weight row 8(r/4) + 4*half + r%4 of the wave's 32, pair lane%32
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int pr = j * 32 + row;
        if (pr >= cnt) continue;
        float* out = p.part + (int64_t)prow[pr] * N;
        const f32x16_t v = acc[j][0] + acc[j][1];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t n = n0 + wv * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (n < N) out[n] = v[r];
        }
    }
}

hipError_t launch_moe_prefill_mxfp4(const MoeArgs& a, int32_t* offs, int32_t* toffs, int32_t* perm,
                                    hipStream_t st) {
    const int P = (int)(a.M * a.topk);
    // direct-to-LDS kernel when K tiles of 256 fit and the scale rows allow
    // 4-byte loads
    const bool dma = a.K % kPdBK == 0 && ((uintptr_t)a.s & 3) == 0;
    // 32-pair tiles (two workgroups per CU); 64-pair tiles (one per CU) were
    // slower at 512 tokens, 48 pairs per expert: 263 vs 241 us
    const int bm = dma ? 32 : kPfBM;
    hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(1024), 0, st, a.ids, P, (int)a.E, bm, offs, toffs, perm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // every expert with pairs needs ceil(count / bm) tiles: at most P / bm + min(E, P)
    const int64_t max_tiles = (P + bm - 1) / bm + (a.E < P ? a.E : P);
    MoeGemmParams p{a.x, a.ldx, a.K, a.w, a.s, (int)a.E, a.N, (int)a.topk, offs, toffs, perm, a.part};
    if (dma) {
        dim3 grid((unsigned)((a.N + kPdBN - 1) / kPdBN), (unsigned)max_tiles);
        hipLaunchKernelGGL(moe_gemm_dma_kernel<32>, grid, dim3(256), 0, st, p);
    } else {
        dim3 grid((unsigned)((a.N + kPfBN - 1) / kPfBN), (unsigned)max_tiles);
        hipLaunchKernelGGL(moe_gemm_kernel, grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace qlin
