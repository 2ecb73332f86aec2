// Internal declarations of the HIP path: device helpers and the host-side
// launchers that api.hip dispatches to.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// ---------------------------------------------------------------------------
// Element access.  A bfloat16 is the upper half of a binary32, so widening is
// a shift (low half of a packed pair) or a mask (high half).
// ---------------------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float widen_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float widen_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i].bits << 16);
}

// Monotone map of binary32 onto uint32: a < b (as floats, NaN above +inf)
// iff key(a) < key(b).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Argmax key: score in the high word, complemented token id in the low word,
// so an unsigned max picks the highest score and, among equal scores, the
// lowest token id.  A zero key means "no candidate" and decodes to -1.
__device__ __forceinline__ uint64_t argmax_key(float score, uint32_t v) {
    return ((uint64_t)orderable(score) << 32) | (uint64_t)(0xffffffffu - v);
}
__device__ __forceinline__ int32_t key_token(uint64_t key) {
    return key == 0 ? -1 : (int32_t)(0xffffffffu - (uint32_t)key);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// exp(x - m) with the log2(e) scale folded into one FMA ahead of v_exp_f32.
__device__ __forceinline__ float exp_shifted(float x, float m_log2e) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(x, 1.4426950408889634f, -m_log2e));
}

// ---------------------------------------------------------------------------
// Workspace header.  Every workspace of the sampler, accept-rate and verify
// entry points begins with these 256 bytes:
//   word 0  private to the kernel that uses the workspace (exit counter)
//   word 1  give-up status: set to 1 by any workgroup whose bounded wait for
//           another workgroup ran out (its outputs are then -1 / NaN and the
//           workspace may be left dirty)
//   word 2  private (the accept-rate row counter)
//   word 3  path flags: kernels only OR bits into it and never read it
// ---------------------------------------------------------------------------
constexpr size_t kWsHeader = 256;
constexpr int kHdrStatus = 1;
constexpr int kHdrPaths = 3;
constexpr uint32_t kPathB1Rebuild = 1u;    // B=1 screen: the norm guess was low, table rebuilt
constexpr uint32_t kPathB1Exchange = 2u;   // B=1: steps settled by the grid-wide per-step exchange
constexpr uint32_t kPathResident = 4u;     // batched sampler: the resident-W2 kernel ran
constexpr uint32_t kPathAcceptCluster = 8u;  // accept rate: the cluster kernel ran
constexpr uint32_t kPathB1Bound = 16u;      // B=1 screen: a precomputed W2 bound replaced the norm stream
constexpr uint32_t kPathB1BoundStale = 32u;  // B=1: the bound's fingerprint did not match W2 (exchange used)
constexpr uint32_t kW2BoundTag = 0x5b0d2a7eu;  // last word of a complete dspark_w2_bound result
constexpr int kW2BoundWords = 8;

__device__ __forceinline__ void mark_gave_up(uint32_t* header) {
    __hip_atomic_store(header + kHdrStatus, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void mark_path(uint32_t* header, uint32_t bit) {
    __hip_atomic_fetch_or(header + kHdrPaths, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll limit of every wait for another workgroup: the kernel's own default
// (a negative value) unless dspark_set_wait_limit set one.
int wait_limit(int kernel_default);

// ---------------------------------------------------------------------------
// Host-side launchers (argument checks already done by the ABI layer).
// ---------------------------------------------------------------------------
size_t accept_rate_workspace(int64_t N, int64_t V);
hipError_t accept_rate_launch(int64_t N, int64_t V, int dtype, const void* d, int64_t ldd, const void* t,
                              int64_t ldt, float* out, void* ws, hipStream_t stream);

size_t head_sample_workspace(int64_t B, int64_t gamma, int64_t V, int64_t r, int dtype);
size_t head_sample_gated_workspace(int64_t B, int64_t gamma, int64_t r, int dtype);
size_t head_sample_rnn_workspace(int64_t B, int64_t gamma, int64_t r, int dtype);
// Wg and Wrg == nullptr: the vanilla Markov head; Wg: the gated head; Wrg and
// Wrc: the RNN head (both on the general path)
hipError_t head_sample_launch(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int dtype, const void* U,
                              const void* h, const void* W1, const void* W2, const void* w_conf, float b_conf,
                              const int32_t* x0, const float* gumbel, const int32_t* force, int32_t* tokens,
                              float* conf, float* survival, float* logits_out, float* bias_out, void* ws,
                              hipStream_t stream, const void* Wg, const void* Wrg, const void* Wrc,
                              const uint32_t* w2_bound = nullptr);
// the weights-only bound of the B = 1 screen (bf16, r = 256): kW2BoundWords words
hipError_t w2_bound_launch(int64_t V, const void* W2, uint32_t* out, hipStream_t stream);

size_t verify_workspace(int64_t B, int64_t gamma, int64_t V);
hipError_t verify_launch(int64_t B, int64_t gamma, int64_t V, int dtype, const void* d, const void* t,
                         const int32_t* x, const int32_t* n_draft, const float* u, const float* G,
                         int32_t* n_accepted, int32_t* next_token, float* accept_prob, void* ws, hipStream_t stream);

size_t prefix_schedule_workspace(int64_t B, int64_t gamma);
hipError_t prefix_schedule_launch(int64_t B, int64_t gamma, const float* conf, const double* sps, int64_t n_sps,
                                  int32_t* prefix_len, float* survival_out, int32_t* order_out, double* theta_out,
                                  int32_t* n_selected_out, void* ws, hipStream_t stream);

}  // namespace dspark
