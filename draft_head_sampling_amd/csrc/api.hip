// C ABI of the draft-head hot path: host-side argument checks, workspace
// queries and dispatch to the kernels.  Every check runs before anything is
// enqueued, and no C++ exception crosses the interface.
#include <atomic>
#include <mutex>

#include "dspark.h"
#include "internal.h"
#include "block_loss.h"

#define DSPARK_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxV = 0x7fffffff;
constexpr int64_t kMaxRank = 1024;      // Markov rank: the gathered rows of W1 live in LDS
constexpr int64_t kMaxSchedPairs = 8192;  // one workgroup sorts all pairs in LDS
constexpr int64_t kMaxRequests = 65535 * 8;  // request groups of 8 along grid.y

bool mul_ok(int64_t a, int64_t b, int64_t limit = INT64_MAX / 16) {
    return a == 0 || b == 0 || (a <= limit / b);
}

dspark_status_t check_workspace(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return DSPARK_OK;
    if (!ws || ws_bytes < need || ((uintptr_t)ws % 256) != 0) return DSPARK_ERR_WORKSPACE;
    return DSPARK_OK;
}

bool sampler_shape_ok(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r) {
    if (B < 0 || B > kMaxRequests || gamma < 0 || V < 1 || V > kMaxV || H < 0 || r < 1 || r > kMaxRank)
        return false;
    return mul_ok(B, gamma) && mul_ok(B * gamma, V) && mul_ok(B * gamma, H) && mul_ok(V, r) &&
           B * gamma <= 0x7fffffff;
}

dspark_status_t hip_status(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

// Poll limit set by dspark_set_wait_limit; negative: each kernel's own default.
std::atomic<int64_t> g_wait_limit{-1};
constexpr int64_t kMaxWaitLimit = (int64_t)1 << 30;

// One thread: copy the give-up status and the path flags of a workspace
// header, then clear the path flags.
__global__ void workspace_status_kernel(uint32_t* header, uint32_t* out) {
    out[0] = __hip_atomic_load(header + dspark::kHdrStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out[1] = __hip_atomic_exchange(header + dspark::kHdrPaths, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

namespace dspark {
int wait_limit(int kernel_default) {
    const int64_t v = g_wait_limit.load(std::memory_order_relaxed);
    return v < 0 ? kernel_default : (int)v;
}
}  // namespace dspark

DSPARK_EXPORT dspark_status_t dspark_set_wait_limit(int64_t polls, int64_t* previous) {
    if (polls > kMaxWaitLimit) return DSPARK_ERR_BAD_SHAPE;
    const int64_t old = g_wait_limit.exchange(polls < 0 ? -1 : polls, std::memory_order_relaxed);
    if (previous) *previous = old;
    return DSPARK_OK;
}

DSPARK_EXPORT dspark_status_t dspark_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* out,
                                                      void* stream) {
    if (!workspace || !out) return DSPARK_ERR_NULL_ARG;
    if (workspace_bytes < dspark::kWsHeader || ((uintptr_t)workspace % 256) != 0) return DSPARK_ERR_WORKSPACE;
    hipLaunchKernelGGL(workspace_status_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(workspace), out);
    return hip_status(hipGetLastError());
}

DSPARK_EXPORT const char* dspark_status_string(dspark_status_t s) {
    switch (s) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_NULL_ARG: return "a required pointer argument is NULL";
        case DSPARK_ERR_BAD_SHAPE: return "a size argument is out of range";
        case DSPARK_ERR_BAD_DTYPE: return "unknown dtype";
        case DSPARK_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case DSPARK_ERR_HIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

DSPARK_EXPORT dspark_status_t dspark_head_sample(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                 int32_t dtype, const void* U, const void* h, const void* W1,
                                                 const void* W2, const void* w_conf, float b_conf, const int32_t* x0,
                                                 const float* gumbel, const int32_t* force, int32_t* tokens,
                                                 float* conf, float* survival, float* logits_out, float* bias_out,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!sampler_shape_ok(B, gamma, V, H, r)) return DSPARK_ERR_BAD_SHAPE;
    if (B == 0 || gamma == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::head_sample_workspace(B, gamma, V, r, dtype));
    if (st != DSPARK_OK) return st;
    if (!U || !W1 || !W2 || !w_conf || !x0 || !tokens || !conf || !survival || (H > 0 && !h))
        return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::head_sample_launch(B, gamma, V, H, r, dtype, U, h, W1, W2, w_conf, b_conf, x0, gumbel,
                                                 force, tokens, conf, survival, logits_out, bias_out, workspace,
                                                 static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr));
}

DSPARK_EXPORT dspark_status_t dspark_head_sample_w2bound(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                         int32_t dtype, const void* U, const void* h, const void* W1,
                                                         const void* W2, const void* w_conf, float b_conf,
                                                         const int32_t* x0, const float* gumbel, const int32_t* force,
                                                         int32_t* tokens, float* conf, float* survival,
                                                         float* logits_out, float* bias_out, const uint32_t* w2_bound,
                                                         void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!sampler_shape_ok(B, gamma, V, H, r)) return DSPARK_ERR_BAD_SHAPE;
    if (B == 0 || gamma == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::head_sample_workspace(B, gamma, V, r, dtype));
    if (st != DSPARK_OK) return st;
    if (!U || !W1 || !W2 || !w_conf || !x0 || !tokens || !conf || !survival || (H > 0 && !h))
        return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::head_sample_launch(B, gamma, V, H, r, dtype, U, h, W1, W2, w_conf, b_conf, x0, gumbel,
                                                 force, tokens, conf, survival, logits_out, bias_out, workspace,
                                                 static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr,
                                                 w2_bound));
}

DSPARK_EXPORT dspark_status_t dspark_w2_bound(int64_t V, int64_t r, int32_t dtype, const void* W2, uint32_t* bound,
                                              void* stream) {
    if (dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (V < 1 || V > kMaxV || r != 256) return DSPARK_ERR_BAD_SHAPE;
    if (!W2 || !bound) return DSPARK_ERR_NULL_ARG;
    if ((uintptr_t)W2 % 16 != 0) return DSPARK_ERR_BAD_SHAPE;  // the screen reads 16-byte pieces
    return hip_status(dspark::w2_bound_launch(V, W2, bound, static_cast<hipStream_t>(stream)));
}

DSPARK_EXPORT dspark_status_t dspark_head_sample_gated(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                       int32_t dtype, const void* U, const void* h, const void* W1,
                                                       const void* W2, const void* w_conf, const void* Wg,
                                                       float b_conf, const int32_t* x0, const float* gumbel,
                                                       const int32_t* force, int32_t* tokens, float* conf,
                                                       float* survival, float* logits_out, float* bias_out,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!sampler_shape_ok(B, gamma, V, H, r) || !mul_ok(r, H + r) || !mul_ok(B * (gamma + 1), r))
        return DSPARK_ERR_BAD_SHAPE;
    if (B == 0 || gamma == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::head_sample_gated_workspace(B, gamma, r, dtype));
    if (st != DSPARK_OK) return st;
    if (!U || !W1 || !W2 || !w_conf || !Wg || !x0 || !tokens || !conf || !survival || (H > 0 && !h))
        return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::head_sample_launch(B, gamma, V, H, r, dtype, U, h, W1, W2, w_conf, b_conf, x0, gumbel,
                                                 force, tokens, conf, survival, logits_out, bias_out, workspace,
                                                 static_cast<hipStream_t>(stream), Wg, nullptr, nullptr));
}

DSPARK_EXPORT dspark_status_t dspark_head_sample_rnn(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                     int32_t dtype, const void* U, const void* h, const void* W1,
                                                     const void* W2, const void* w_conf, const void* Wrg,
                                                     const void* Wrc, float b_conf, const int32_t* x0,
                                                     const float* gumbel, const int32_t* force, int32_t* tokens,
                                                     float* conf, float* survival, float* logits_out,
                                                     float* bias_out, void* workspace, size_t workspace_bytes,
                                                     void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!sampler_shape_ok(B, gamma, V, H, r) || !mul_ok(r, 2 * r + H) || !mul_ok(B * (2 * gamma + 2), r))
        return DSPARK_ERR_BAD_SHAPE;
    if (B == 0 || gamma == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::head_sample_rnn_workspace(B, gamma, r, dtype));
    if (st != DSPARK_OK) return st;
    if (!U || !W1 || !W2 || !w_conf || !Wrg || !Wrc || !x0 || !tokens || !conf || !survival || (H > 0 && !h))
        return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::head_sample_launch(B, gamma, V, H, r, dtype, U, h, W1, W2, w_conf, b_conf, x0, gumbel,
                                                 force, tokens, conf, survival, logits_out, bias_out, workspace,
                                                 static_cast<hipStream_t>(stream), nullptr, Wrg, Wrc));
}

DSPARK_EXPORT size_t dspark_head_sample_rnn_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                           int32_t dtype) {
    if (!sampler_shape_ok(B, gamma, V, H, r) || !mul_ok(r, 2 * r + H) || !mul_ok(B * (2 * gamma + 2), r)) return 0;
    return dspark::head_sample_rnn_workspace(B, gamma, r, dtype);
}

DSPARK_EXPORT dspark_status_t dspark_accept_rate(int64_t N, int64_t V, int32_t dtype, const void* draft,
                                                 int64_t ld_draft, const void* target, int64_t ld_target,
                                                 float* accept_rate, void* workspace, size_t workspace_bytes,
                                                 void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (N < 0 || V < 1 || V > kMaxV || ld_draft < V || ld_target < V) return DSPARK_ERR_BAD_SHAPE;
    if (!mul_ok(N, ld_draft) || !mul_ok(N, ld_target)) return DSPARK_ERR_BAD_SHAPE;
    if (N == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::accept_rate_workspace(N, V));
    if (st != DSPARK_OK) return st;
    if (!draft || !target || !accept_rate) return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::accept_rate_launch(N, V, dtype, draft, ld_draft, target, ld_target, accept_rate,
                                                 workspace, static_cast<hipStream_t>(stream)));
}

DSPARK_EXPORT dspark_status_t dspark_prefix_schedule(int64_t B, int64_t gamma, const float* conf, const double* sps,
                                                     int64_t n_sps, int32_t* prefix_len, float* survival_out,
                                                     int32_t* order_out, double* theta_out, int32_t* n_selected_out,
                                                     void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 1 || B > kMaxSchedPairs || gamma < 0 || n_sps < B || !mul_ok(B, gamma) || B * gamma > kMaxSchedPairs)
        return DSPARK_ERR_BAD_SHAPE;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::prefix_schedule_workspace(B, gamma));
    if (st != DSPARK_OK) return st;
    if (!sps || !prefix_len || (gamma > 0 && !conf)) return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::prefix_schedule_launch(B, gamma, conf, sps, n_sps, prefix_len, survival_out, order_out,
                                                     theta_out, n_selected_out, workspace,
                                                     static_cast<hipStream_t>(stream)));
}

namespace {
constexpr int64_t kMaxVerifyRequests = 65535;  // grid.y of the sampling launch
constexpr int64_t kMaxVerifyGamma = 4096;      // the sample's position travels in 16 bits

bool verify_shape_ok(int64_t B, int64_t gamma, int64_t V) {
    return B >= 0 && B <= kMaxVerifyRequests && gamma >= 0 && gamma <= kMaxVerifyGamma && V >= 1 && V <= kMaxV &&
           mul_ok(B * (gamma + 1), V);
}
}  // namespace

DSPARK_EXPORT dspark_status_t dspark_verify(int64_t B, int64_t gamma, int64_t V, int32_t dtype, const void* draft,
                                            const void* target, const int32_t* draft_tokens, const int32_t* n_draft,
                                            const float* uniforms, const float* gumbel, int32_t* n_accepted,
                                            int32_t* next_token, float* accept_prob, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!verify_shape_ok(B, gamma, V)) return DSPARK_ERR_BAD_SHAPE;
    if (B == 0) return DSPARK_OK;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::verify_workspace(B, gamma, V));
    if (st != DSPARK_OK) return st;
    if (!target || !gumbel || !n_accepted || !next_token || (gamma > 0 && (!draft || !draft_tokens || !uniforms)))
        return DSPARK_ERR_NULL_ARG;
    return hip_status(dspark::verify_launch(B, gamma, V, dtype, draft, target, draft_tokens, n_draft, uniforms, gumbel,
                                            n_accepted, next_token, accept_prob, workspace,
                                            static_cast<hipStream_t>(stream)));
}

DSPARK_EXPORT size_t dspark_verify_workspace_size(int64_t B, int64_t gamma, int64_t V, int32_t) {
    if (!verify_shape_ok(B, gamma, V)) return 0;
    return dspark::verify_workspace(B, gamma, V);
}

DSPARK_EXPORT size_t dspark_head_sample_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                       int32_t dtype) {
    if (!sampler_shape_ok(B, gamma, V, H, r)) return 0;
    return dspark::head_sample_workspace(B, gamma, V, r, dtype);
}

DSPARK_EXPORT size_t dspark_head_sample_gated_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H,
                                                             int64_t r, int32_t dtype) {
    if (!sampler_shape_ok(B, gamma, V, H, r) || !mul_ok(r, H + r) || !mul_ok(B * (gamma + 1), r)) return 0;
    return dspark::head_sample_gated_workspace(B, gamma, r, dtype);
}

DSPARK_EXPORT size_t dspark_accept_rate_workspace_size(int64_t N, int64_t V, int32_t) {
    if (N < 0 || V < 1 || V > kMaxV) return 0;
    return dspark::accept_rate_workspace(N, V);
}

DSPARK_EXPORT size_t dspark_prefix_schedule_workspace_size(int64_t B, int64_t gamma) {
    if (B < 1 || B > kMaxSchedPairs || gamma < 0 || !mul_ok(B, gamma) || B * gamma > kMaxSchedPairs) return 0;
    return dspark::prefix_schedule_workspace(B, gamma);
}

namespace {
constexpr int64_t kMaxLossChunks = 65535;  // vocabulary chunks of 512 rows along grid.y

bool block_loss_dims_ok(int64_t N, int64_t gamma, int64_t V, int64_t H) {
    if (N < 0 || gamma < 0 || V < 1 || V > kMaxLossChunks * 512 || H < 0) return false;
    return mul_ok(N, gamma) && N * gamma <= 0x7fffffff && mul_ok(N * gamma, V) && mul_ok(N * gamma, H);
}
}  // namespace

DSPARK_EXPORT size_t dspark_block_loss_workspace_size(int64_t N, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                      int32_t) {
    if (!block_loss_dims_ok(N, gamma, V, H) || r < 1) return 0;
    return dspark::block_loss_workspace(N * gamma, V);
}

DSPARK_EXPORT dspark_status_t dspark_block_loss(int64_t N, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                int32_t dtype, const void* U, const void* t, const void* h,
                                                const void* W1, const void* W2, const void* w_conf, float b_conf,
                                                const int32_t* xp, const int32_t* y, const float* mask, float decay,
                                                float a_ce, float a_l1, float a_conf, float* ce, float* l1,
                                                float* conf, float* bce, float* loss, void* workspace,
                                                size_t workspace_bytes, void* stream) {
    if (dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!block_loss_dims_ok(N, gamma, V, H) || !(decay > 0.f)) return DSPARK_ERR_BAD_SHAPE;
    const int64_t M = N * gamma;
    if (!loss) return DSPARK_ERR_NULL_ARG;
    if (M > 0 && (!U || !t || !W1 || !W2 || !w_conf || !xp || !y || !ce || !l1 || !conf || !bce || (H > 0 && !h)))
        return DSPARK_ERR_NULL_ARG;
    dspark_status_t st = check_workspace(workspace, workspace_bytes, dspark::block_loss_workspace(M, V));
    if (st != DSPARK_OK) return st;
    if (!dspark::block_loss_shape_ok(r, W1, W2, workspace)) return DSPARK_ERR_BAD_SHAPE;
    return hip_status(dspark::block_loss_launch(N, gamma, V, H, U, t, h, W1, W2, w_conf, b_conf, xp, y, mask, decay,
                                                a_ce, a_l1, a_conf, ce, l1, conf, bce, loss, workspace,
                                                static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// Allocation-free variant of dspark_head_sample for callers that cannot
// allocate (graph capture, tight serving loops): its workspace is a static
// device array of kScratchBytes per GPU, held until the process ends.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;
// In host code `scratch` names a host-side stand-in; kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kScratchMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kScratchMaxDevices];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot& s = g_scratch[dev];
    std::call_once(s.once, [&s]() {
        void* p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        s.ptr = s.err == hipSuccess ? p : nullptr;
    });
    if (s.err != hipSuccess) return s.err;
    if (s.ptr == nullptr) return hipErrorInvalidSymbol;
    *out = s.ptr;
    return hipSuccess;
}

// Zero n bytes (a multiple of 16) with vector stores: the kernels expect a
// zero-filled workspace, and the array keeps whatever the last call left.
__global__ void zero_words(uint4* p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

DSPARK_EXPORT dspark_status_t dspark_head_sample_noalloc(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                         int32_t dtype, const void* U, const void* h, const void* W1,
                                                         const void* W2, const void* w_conf, float b_conf,
                                                         const int32_t* x0, const float* gumbel, const int32_t* force,
                                                         int32_t* tokens, float* conf, float* survival,
                                                         float* logits_out, float* bias_out, void* stream) {
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_BAD_DTYPE;
    if (!sampler_shape_ok(B, gamma, V, H, r)) return DSPARK_ERR_BAD_SHAPE;
    if (B == 0 || gamma == 0) return DSPARK_OK;
    const size_t need = (dspark::head_sample_workspace(B, gamma, V, r, dtype) + 255) / 256 * 256;
    if (need > kScratchBytes) return DSPARK_ERR_WORKSPACE;
    if (!U || !W1 || !W2 || !w_conf || !x0 || !tokens || !conf || !survival || (H > 0 && !h))
        return DSPARK_ERR_NULL_ARG;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return DSPARK_ERR_HIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n16 = (int64_t)(need / 16);
    const int64_t blocks = (n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero_words, dim3((uint32_t)blocks), dim3(256), 0, st, static_cast<uint4*>(ws), n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return DSPARK_ERR_HIP;
    return hip_status(dspark::head_sample_launch(B, gamma, V, H, r, dtype, U, h, W1, W2, w_conf, b_conf, x0, gumbel,
                                                 force, tokens, conf, survival, logits_out, bias_out, ws, st, nullptr,
                                                 nullptr, nullptr));
}
