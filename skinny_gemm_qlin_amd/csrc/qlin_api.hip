// qlin_api.hip -- the extern "C" entry points declared in include/qlin.h.
//
// Each entry point validates every host-visible argument (pointers, shapes,
// pitches, alignment, flags) and returns a QLIN_ERR_* code before anything is
// enqueued; only then does it launch the kernels on the caller's stream.
// No allocation, no synchronisation.  The only state is the per-device
// address of the scratch array behind qlin_moe_mxfp4_noalloc.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qlin.h"
#include "qlin_launch.hpp"

namespace {

inline bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p) % a != 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? QLIN_OK : QLIN_ERR_LAUNCH; }

constexpr int64_t kMaxKInt8 = 131072;  // K * 127 * 128 < 2^31: int32 accumulation is exact
constexpr int64_t kMaxKFp8 = 1 << 24;  // keeps the quantiser's 32-bit vector indexes in range
constexpr int64_t kMaxKBlkGeneral = 32768;  // the general block GEMV stages K/32 x 32 scale bytes in LDS
constexpr int64_t kMaxEPrefill = 1024;      // the pair sort counts experts in one workgroup's LDS
constexpr int64_t kFusedI8MaxK = 8192;      // the one-launch INT8 layer keeps the token's codes in LDS

}  // namespace

extern "C" {

const char* qlin_status_str(int status) {
    switch (status) {
        case QLIN_OK: return "QLIN_OK";
        case QLIN_ERR_NULL: return "QLIN_ERR_NULL: a required pointer is NULL";
        case QLIN_ERR_SHAPE: return "QLIN_ERR_SHAPE: M, N, K or topk outside the supported range";
        case QLIN_ERR_STRIDE: return "QLIN_ERR_STRIDE: a row pitch is smaller than its row";
        case QLIN_ERR_ALIGN: return "QLIN_ERR_ALIGN: a pointer or row pitch is not aligned";
        case QLIN_ERR_WORKSPACE: return "QLIN_ERR_WORKSPACE: workspace missing or too small";
        case QLIN_ERR_ARG: return "QLIN_ERR_ARG: unknown flag value";
        case QLIN_ERR_LAUNCH: return "QLIN_ERR_LAUNCH: HIP kernel launch failed";
        default: return "QLIN_ERR_UNKNOWN";
    }
}

int qlin_version(void) { return 100; }  // 0.1.0

int qlin_act_quant_i8(const void* x, int64_t ldx, int64_t M, int64_t K,
                      int8_t* xq, int64_t ldxq, float* xs, void* stream) {
    if (!x || !xq || !xs) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || K < 16 || K % 16 != 0 || K > kMaxKInt8) return QLIN_ERR_SHAPE;
    if (ldx < K || ldxq < K) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(xq, 16) || ldxq % 16 != 0 || misaligned(xs, 4))
        return QLIN_ERR_ALIGN;
    qlin::ActQuantI8Args a{(const uint16_t*)x, ldx, M, K, xq, ldxq, xs};
    return launch_status(qlin::launch_act_quant_i8(a, (hipStream_t)stream));
}

int qlin_gemv_i8(const int8_t* xq, int64_t ldxq, const float* xs, int xs_per_token,
                 int64_t M, int64_t K, const int8_t* w, int64_t ldw, int64_t N,
                 const float* ws, int ws_per_row, const void* bias,
                 void* y, int64_t ldy, int out_kind, void* stream) {
    if (out_kind != 0 && out_kind != 1) return QLIN_ERR_ARG;
    if ((xs_per_token != 0 && xs_per_token != 1) || (ws_per_row != 0 && ws_per_row != 1)) return QLIN_ERR_ARG;
    if (!xq || !w || !y) return QLIN_ERR_NULL;
    if (out_kind == 0 && (!xs || !ws)) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < 16 || K % 16 != 0 || K > kMaxKInt8) return QLIN_ERR_SHAPE;
    if (ldxq < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(xq, 16) || ldxq % 16 != 0 || misaligned(w, 16) || ldw % 16 != 0) return QLIN_ERR_ALIGN;
    if (misaligned(y, out_kind == 1 ? 4 : 2) || (xs && misaligned(xs, 4)) || (ws && misaligned(ws, 4)) ||
        (bias && misaligned(bias, 2)))
        return QLIN_ERR_ALIGN;
    qlin::I8Args a{xq, ldxq, xs, xs_per_token ? 1 : 0, M, K, w, ldw, N, ws, ws_per_row ? 1 : 0,
                   (const uint16_t*)bias, y, ldy, out_kind};
    return launch_status(qlin::launch_gemv_i8(a, (hipStream_t)stream));
}

int qlin_linear_i8(const void* x, int64_t ldx, int64_t M, int64_t K,
                   const int8_t* w, int64_t ldw, int64_t N, const float* ws, int ws_per_row, const void* bias,
                   int8_t* xq, int64_t ldxq, float* xs, void* y, int64_t ldy, void* stream) {
    if (ws_per_row != 0 && ws_per_row != 1) return QLIN_ERR_ARG;
    if (!x || !w || !ws || !xq || !xs || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < 16 || K % 16 != 0 || K > kMaxKInt8) return QLIN_ERR_SHAPE;
    if (ldx < K || ldxq < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(xq, 16) || ldxq % 16 != 0 || misaligned(xs, 4) ||
        misaligned(w, 16) || ldw % 16 != 0 || misaligned(ws, 4) || misaligned(y, 2) || (bias && misaligned(bias, 2)))
        return QLIN_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    qlin::ActQuantI8Args q{(const uint16_t*)x, ldx, M, K, xq, ldxq, xs};
    qlin::I8Args a{xq, ldxq, xs, 1, M, K, w, ldw, N, ws, ws_per_row ? 1 : 0, (const uint16_t*)bias, y, ldy, 0};
    if (M == 1 && K <= kFusedI8MaxK) return launch_status(qlin::launch_linear_i8_fused(q, a, st));
    if (qlin::launch_act_quant_i8(q, st) != hipSuccess) return QLIN_ERR_LAUNCH;
    return launch_status(qlin::launch_gemv_i8(a, st));
}

int qlin_gemv_fp8(const void* x, int64_t ldx, int64_t M, int64_t K,
                  const uint8_t* w, int64_t ldw, int64_t N, const float* ws, int ws_per_row,
                  void* y, int64_t ldy, void* stream) {
    if (ws_per_row != 0 && ws_per_row != 1) return QLIN_ERR_ARG;
    if (!x || !w || !ws || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < 16 || K % 16 != 0) return QLIN_ERR_SHAPE;
    if (ldx < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(w, 16) || ldw % 16 != 0 || misaligned(ws, 4) ||
        misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    qlin::F8Args a{(const uint16_t*)x, ldx, M, K, w, ldw, N, ws, ws_per_row ? 1 : 0, (uint16_t*)y, ldy};
    return launch_status(qlin::launch_gemv_fp8(a, (hipStream_t)stream));
}

int qlin_act_quant_fp8(const void* x, int64_t ldx, int64_t M, int64_t K, int fmt, int per_token,
                       uint8_t* xq, int64_t ldxq, float* xs, void* stream) {
    if ((fmt != QLIN_FMT_E4M3 && fmt != QLIN_FMT_E5M2) || (per_token != 0 && per_token != 1)) return QLIN_ERR_ARG;
    if (!x || !xq || !xs) return QLIN_ERR_NULL;
    if (M < 1 || M > (per_token ? QLIN_MAX_M_PREFILL : QLIN_MAX_M) || K < 16 || K % 16 != 0 || K > kMaxKFp8)
        return QLIN_ERR_SHAPE;
    if (ldx < K || ldxq < K) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(xq, 16) || ldxq % 16 != 0 || misaligned(xs, 4))
        return QLIN_ERR_ALIGN;
    qlin::ActQuantF8Args a{(const uint16_t*)x, ldx, M, K, fmt, per_token, xq, ldxq, xs};
    return launch_status(qlin::launch_act_quant_fp8(a, (hipStream_t)stream));
}

int qlin_gemv_fp8_w8a8(const uint8_t* xq, int64_t ldxq, const float* xs, int xs_per_token, int x_fmt,
                       int64_t M, int64_t K, const uint8_t* w, int64_t ldw, int64_t N,
                       const float* ws, int ws_per_row, int w_fmt, void* y, int64_t ldy, void* stream) {
    if ((x_fmt != QLIN_FMT_E4M3 && x_fmt != QLIN_FMT_E5M2) || (w_fmt != QLIN_FMT_E4M3 && w_fmt != QLIN_FMT_E5M2))
        return QLIN_ERR_ARG;
    if ((xs_per_token != 0 && xs_per_token != 1) || (ws_per_row != 0 && ws_per_row != 1)) return QLIN_ERR_ARG;
    if (!xq || !xs || !w || !ws || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < 16 || K % 16 != 0 || K > kMaxKFp8) return QLIN_ERR_SHAPE;
    if (ldxq < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(xq, 16) || ldxq % 16 != 0 || misaligned(w, 16) || ldw % 16 != 0 || misaligned(xs, 4) ||
        misaligned(ws, 4) || misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    qlin::W8A8F8Args a{xq, ldxq, xs, xs_per_token ? 1 : 0, x_fmt, M, K, w, ldw, N,
                       ws, ws_per_row ? 1 : 0, w_fmt, (uint16_t*)y, ldy};
    return launch_status(qlin::launch_gemv_fp8_w8a8(a, (hipStream_t)stream));
}

int qlin_gemv_fp8_blk(const void* x, int64_t ldx, int64_t M, int64_t K,
                      const uint8_t* w, int64_t ldw, int64_t N, const uint8_t* ws,
                      uint8_t* xq, uint8_t* xs, void* y, int64_t ldy, void* stream) {
    if (!x || !w || !ws || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < 128 || K % 128 != 0) return QLIN_ERR_SHAPE;
    const bool fused = M == 1 && K <= qlin::kBlkFusedMaxK;  // one launch; xq / xs then optional
    if (!fused && (!xq || !xs)) return QLIN_ERR_NULL;
    if (ldx < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(w, 16) || ldw % 16 != 0 || (xq && misaligned(xq, 16)) ||
        misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    qlin::BlkQuantArgs qa{(const uint16_t*)x, ldx, M, K, xq, xs};
    qlin::BlkArgs a{xq, xs, M, K, w, ldw, N, ws, (uint16_t*)y, ldy};
    if (fused) return launch_status(qlin::launch_gemv_fp8_blk_fq(qa, a, st));
    hipError_t e = qlin::launch_blk_act_quant(qa, st);
    if (e != hipSuccess) return QLIN_ERR_LAUNCH;
    return launch_status(qlin::launch_gemv_fp8_blk(a, st));
}

int qlin_gemv_fp8_blk_ex(const void* x, int64_t ldx, int64_t M, int64_t K,
                         const uint8_t* w, int64_t ldw, int64_t N, const uint8_t* ws,
                         int64_t block_n, int64_t block_k,
                         uint8_t* xq, uint8_t* xs, void* y, int64_t ldy, void* stream) {
    if (!x || !w || !ws || !xq || !xs || !y) return QLIN_ERR_NULL;
    if (block_n < 1 || block_k < 32 || block_k % 32 != 0) return QLIN_ERR_SHAPE;
    if (block_n == 128 && block_k == 128)  // the tested configuration keeps its own kernels
        return qlin_gemv_fp8_blk(x, ldx, M, K, w, ldw, N, ws, xq, xs, y, ldy, stream);
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || K < block_k || K % block_k != 0 || K > kMaxKBlkGeneral)
        return QLIN_ERR_SHAPE;
    if (ldx < K || ldw < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(w, 16) || ldw % 16 != 0 || misaligned(xq, 16) ||
        misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    qlin::BlkQuantArgs qa{(const uint16_t*)x, ldx, M, K, xq, xs};
    if (qlin::launch_blkg_act_quant(qa, block_k, st) != hipSuccess) return QLIN_ERR_LAUNCH;
    qlin::BlkArgs a{xq, xs, M, K, w, ldw, N, ws, (uint16_t*)y, ldy};
    if (M > QLIN_MAX_M && K % 128 == 0)  // prefill: one GEMM over all tokens
        return launch_status(qlin::launch_gemm_fp8_blkg(a, block_n, block_k, st));
    // the matrix-core kernel over a grid of 16-token blocks
    return launch_status(qlin::launch_gemv_fp8_blkg(a, block_n, block_k, st));
}

size_t qlin_moe_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t topk, int64_t E) {
    if (M < 1 || N < 1 || topk < 1 || E < 1) return 0;
    const size_t b = ((size_t)M * (size_t)topk * (size_t)N * sizeof(float) + 255) & ~(size_t)255;
    if (M <= QLIN_MAX_M) return b;
    // prefill: + pair offsets [E+1], tile offsets [E+1], pair order [M*topk] (int32)
    const size_t s = ((size_t)(2 * (E + 1) + M * topk) * sizeof(int32_t) + 255) & ~(size_t)255;
    return b + s;
}

}  // extern "C"

namespace {

// Argument checks of qlin_moe_mxfp4 other than the workspace.
int moe_mxfp4_check(const void* x, int64_t ldx, int64_t M, int64_t K, const uint8_t* w_fp4,
                    const uint8_t* s_ue8m0, int64_t E, int64_t N, const int32_t* topk_ids, const float* topk_w,
                    int64_t topk, const void* y, int64_t ldy) {
    if (!x || !w_fp4 || !s_ue8m0 || !topk_ids || !topk_w || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M_PREFILL || N < 1 || E < 1 || K < 32 || K % 32 != 0 || K > 30720 || topk < 1 ||
        topk > 16)
        return QLIN_ERR_SHAPE;
    if (M > QLIN_MAX_M && E > kMaxEPrefill) return QLIN_ERR_SHAPE;
    if (ldx < K || ldy < N) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(w_fp4, 16) || misaligned(topk_ids, 4) ||
        misaligned(topk_w, 4) || misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    return QLIN_OK;
}

int moe_mxfp4_launch(const void* x, int64_t ldx, int64_t M, int64_t K, const uint8_t* w_fp4,
                     const uint8_t* s_ue8m0, int64_t E, int64_t N, const int32_t* topk_ids, const float* topk_w,
                     int64_t topk, void* y, int64_t ldy, void* workspace, hipStream_t stream) {
    const size_t part_bytes = ((size_t)M * topk * N * sizeof(float) + 255) & ~(size_t)255;
    qlin::MoeArgs a{(const uint16_t*)x, ldx, M, K, w_fp4, s_ue8m0, E, N, topk_ids, topk_w, topk,
                    (uint16_t*)y, ldy, (float*)workspace, (int32_t*)((char*)workspace + part_bytes)};
    return launch_status(qlin::launch_moe_mxfp4(a, stream));
}

// Workspace of qlin_moe_mxfp4_noalloc: one copy per GPU, alive until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): it passes the device address
// looked up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[QLIN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device ordinal; null until looked up

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream), looked up with that device current.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int qlin_moe_mxfp4(const void* x, int64_t ldx, int64_t M, int64_t K,
                   const uint8_t* w_fp4, const uint8_t* s_ue8m0, int64_t E, int64_t N,
                   const int32_t* topk_ids, const float* topk_w, int64_t topk,
                   void* y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
    const int st = moe_mxfp4_check(x, ldx, M, K, w_fp4, s_ue8m0, E, N, topk_ids, topk_w, topk, y, ldy);
    if (st != QLIN_OK) return st;
    if (!workspace || workspace_bytes < qlin_moe_mxfp4_workspace_bytes(M, N, topk, E)) return QLIN_ERR_WORKSPACE;
    if (misaligned(workspace, 16)) return QLIN_ERR_ALIGN;
    return moe_mxfp4_launch(x, ldx, M, K, w_fp4, s_ue8m0, E, N, topk_ids, topk_w, topk, y, ldy, workspace,
                            (hipStream_t)stream);
}

int qlin_moe_mxfp4_noalloc(const void* x, int64_t ldx, int64_t M, int64_t K,
                           const uint8_t* w_fp4, const uint8_t* s_ue8m0, int64_t E, int64_t N,
                           const int32_t* topk_ids, const float* topk_w, int64_t topk,
                           void* y, int64_t ldy, void* stream) {
    const int st = moe_mxfp4_check(x, ldx, M, K, w_fp4, s_ue8m0, E, N, topk_ids, topk_w, topk, y, ldy);
    if (st != QLIN_OK) return st;
    if (qlin_moe_mxfp4_workspace_bytes(M, N, topk, E) > (size_t)QLIN_NOALLOC_SCRATCH_BYTES)
        return QLIN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (scratch_for_stream((hipStream_t)stream, &ws) != hipSuccess) return QLIN_ERR_LAUNCH;
    return moe_mxfp4_launch(x, ldx, M, K, w_fp4, s_ue8m0, E, N, topk_ids, topk_w, topk, y, ldy, ws,
                            (hipStream_t)stream);
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t qlin_moe_ffn_mxfp4_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk, int64_t E) {
    if (M < 1 || H < 1 || I < 1 || topk < 1 || E < 1) return 0;
    return round256((size_t)M * E * sizeof(float)) + round256((size_t)M * topk * I * sizeof(uint16_t)) +
           round256((size_t)M * topk * H * sizeof(float));
}

int qlin_moe_ffn_mxfp4(const void* x, int64_t ldx, int64_t M, int64_t H,
                       const void* wr, int64_t E, int64_t topk,
                       const uint8_t* w13, const uint8_t* s13, int64_t I,
                       const uint8_t* w2, const uint8_t* s2,
                       float alpha, float limit,
                       int32_t* topk_ids, float* topk_w,
                       void* y, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !wr || !w13 || !s13 || !w2 || !s2 || !topk_ids || !topk_w || !y) return QLIN_ERR_NULL;
    if (M < 1 || M > QLIN_MAX_M || E < 1 || E > 1024 || topk < 1 || topk > 16 || topk > E)
        return QLIN_ERR_SHAPE;
    if (H < 32 || H % 32 != 0 || H > 30720 || I < 32 || I % 32 != 0 || I > 30720) return QLIN_ERR_SHAPE;
    if (ldx < H || ldy < H) return QLIN_ERR_STRIDE;
    if (misaligned(x, 16) || ldx % 8 != 0 || misaligned(wr, 16) || misaligned(w13, 16) ||
        misaligned(w2, 16) || misaligned(topk_ids, 4) || misaligned(topk_w, 4) || misaligned(y, 2))
        return QLIN_ERR_ALIGN;
    if (!workspace || workspace_bytes < qlin_moe_ffn_mxfp4_workspace_bytes(M, H, I, topk, E))
        return QLIN_ERR_WORKSPACE;
    if (misaligned(workspace, 16)) return QLIN_ERR_ALIGN;
    char* ws = (char*)workspace;
    float* logits = (float*)ws;
    uint16_t* act = (uint16_t*)(ws + round256((size_t)M * E * sizeof(float)));
    float* part = (float*)((char*)act + round256((size_t)M * topk * I * sizeof(uint16_t)));
    qlin::MoeFfnArgs a{(const uint16_t*)x, ldx, M, H, (const uint16_t*)wr, E, topk, w13, s13, I, w2, s2,
                       alpha, limit, topk_ids, topk_w, (uint16_t*)y, ldy, logits, act, part};
    return launch_status(qlin::launch_moe_ffn_mxfp4(a, (hipStream_t)stream));
}

}  // extern "C"
