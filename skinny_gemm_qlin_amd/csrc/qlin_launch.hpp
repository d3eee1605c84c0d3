// qlin_launch.hpp -- internal interface between the C-ABI layer (qlin_api.hip)
// and the kernel translation units.  Argument structs carry validated,
// already-normalised arguments (broadcast scales have step 0).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlin {

struct ActQuantI8Args {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t K;
    int8_t* xq; int64_t ldxq; float* xs;
};

struct ActQuantF8Args {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t K; int fmt; int per_token;
    uint8_t* xq; int64_t ldxq; float* xs;
};

struct W8A8F8Args {
    const uint8_t* xq; int64_t ldxq; const float* xs; int xs_step; int x_fmt;
    int64_t M; int64_t K; const uint8_t* w; int64_t ldw; int64_t N;
    const float* ws; int ws_step; int w_fmt; uint16_t* y; int64_t ldy;
};

struct I8Args {
    const int8_t* xq; int64_t ldxq; const float* xs; int xs_step;
    int64_t M; int64_t K; const int8_t* w; int64_t ldw; int64_t N;
    const float* ws; int ws_step; const uint16_t* bias; void* y; int64_t ldy; int out_kind;
};

struct F8Args {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t K;
    const uint8_t* w; int64_t ldw; int64_t N; const float* ws; int ws_step;
    uint16_t* y; int64_t ldy;
};

struct BlkQuantArgs {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t K; uint8_t* xq; uint8_t* xs;
};

struct BlkArgs {
    const uint8_t* xq; const uint8_t* xs; int64_t M; int64_t K;
    const uint8_t* w; int64_t ldw; int64_t N; const uint8_t* ws; uint16_t* y; int64_t ldy;
};

struct MoeArgs {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t K;
    const uint8_t* w; const uint8_t* s; int64_t E; int64_t N;
    const int32_t* ids; const float* gw; int64_t topk;
    uint16_t* y; int64_t ldy; float* part;
    int32_t* sort;  // M > 16: pair offsets [E+1], tile offsets [E+1], pair order [M*topk]
};

hipError_t launch_act_quant_i8(const ActQuantI8Args& a, hipStream_t st);
hipError_t launch_gemv_i8(const I8Args& a, hipStream_t st);
// quantiser + GEMV in one launch (M = 1, K <= 8192); q.xq / q.xs may be null
hipError_t launch_linear_i8_fused(const ActQuantI8Args& q, const I8Args& a, hipStream_t st);
hipError_t launch_gemv_fp8(const F8Args& a, hipStream_t st);
hipError_t launch_act_quant_fp8(const ActQuantF8Args& a, hipStream_t st);
hipError_t launch_gemv_fp8_w8a8(const W8A8F8Args& a, hipStream_t st);
hipError_t launch_blk_act_quant(const BlkQuantArgs& a, hipStream_t st);
hipError_t launch_gemv_fp8_blk(const BlkArgs& a, hipStream_t st);
// act quant + GEMV in one launch (M = 1, K <= kBlkFusedMaxK)
constexpr int64_t kBlkFusedMaxK = 32768;
hipError_t launch_gemv_fp8_blk_fq(const BlkQuantArgs& q, const BlkArgs& a, hipStream_t st);
// any block shape (block_k a multiple of 32), M <= 16 per launch
hipError_t launch_blkg_act_quant(const BlkQuantArgs& a, int64_t bk, hipStream_t st);
hipError_t launch_gemv_fp8_blkg(const BlkArgs& a, int64_t bn, int64_t bk, hipStream_t st);
hipError_t launch_moe_mxfp4(const MoeArgs& a, hipStream_t st);
hipError_t launch_moe_prefill_mxfp4(const MoeArgs& a, int32_t* offs, int32_t* toffs, int32_t* perm, hipStream_t st);

// prefill GEMM (M > 16), called by the launchers above
hipError_t launch_gemm_i8(const I8Args& a, hipStream_t st);
hipError_t launch_gemm_fp8(const F8Args& a, hipStream_t st);
hipError_t launch_gemm_fp8_w8a8(const W8A8F8Args& a, hipStream_t st);
hipError_t launch_gemm_fp8_blk(const BlkArgs& a, hipStream_t st);
hipError_t launch_gemm_fp8_blkg(const BlkArgs& a, int64_t bn, int64_t bk, hipStream_t st);

struct MoeFfnArgs {
    const uint16_t* x; int64_t ldx; int64_t M; int64_t H;
    const uint16_t* wr; int64_t E; int64_t topk;
    const uint8_t* w13; const uint8_t* s13; int64_t I;
    const uint8_t* w2; const uint8_t* s2;
    float alpha; float limit;
    int32_t* ids; float* gw; uint16_t* y; int64_t ldy;
    float* logits; uint16_t* act; float* part;  // workspace regions
};

hipError_t launch_router(const uint16_t* x, int64_t ldx, int64_t M, int64_t H, const uint16_t* wr, int64_t E,
                         float* logits, hipStream_t st);
hipError_t launch_topk_softmax(const float* logits, int64_t M, int64_t E, int64_t topk, int32_t* ids, float* gw,
                               hipStream_t st);
hipError_t launch_moe_ffn_mxfp4(const MoeFfnArgs& a, hipStream_t st);

}  // namespace qlin
