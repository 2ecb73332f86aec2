// Analytic accept rate, paper eq. 8 ("基于 DSpark 的投机解码训练框架原理与实现",
// wangjunjian.com, section 3.3):
//     c*_n = 1 - 1/2 * || softmax(d_n) - softmax(t_n) ||_1
// an HBM-bound two-pass reduction over each row pair.
//
// Pass 1 keeps a running (max, sum of exp(x - max)) per thread for both rows,
// folding each loaded vector in with one rescale; the workgroup then merges
// the per-thread pairs.  Pass 2 re-reads the row pair and accumulates
// |p - q| with the row statistics.  All sums are binary32, reduced in a fixed
// order, so results are bitwise reproducible.
#include "internal.h"

namespace dspark {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 512;

template <typename T>
struct Vec;
template <>
struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, int64_t i, float (&x)[4]) {
        float4 r = *reinterpret_cast<const float4*>(p + i);
        x[0] = r.x, x[1] = r.y, x[2] = r.z, x[3] = r.w;
    }
};
template <>
struct Vec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void load(const bf16_t* p, int64_t i, float (&x)[8]) {
        uint4 r = *reinterpret_cast<const uint4*>(p + i);
        x[0] = widen_lo(r.x), x[1] = widen_hi(r.x), x[2] = widen_lo(r.y), x[3] = widen_hi(r.y);
        x[4] = widen_lo(r.z), x[5] = widen_hi(r.z), x[6] = widen_lo(r.w), x[7] = widen_hi(r.w);
    }
};

// Fold n values into a running (m, s): s <- s * e^(m - m') + sum e^(x - m').
template <int N>
__device__ __forceinline__ void fold(float& m, float& s, const float (&x)[N]) {
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
    const float mn = fmaxf(m, bm);
    const float mnl = mn * kLog2e;
    float acc = s * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -mnl));
#pragma unroll
    for (int i = 0; i < N; ++i) acc += exp_shifted(x[i], mnl);
    s = acc;
    m = mn;
}

__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    const float a = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * kLog2e);
    const float b = (m2 == -INFINITY) ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
    m = mn;
    s = a + b;
}

template <int NT>
__device__ void block_merge(float& m, float& s, float* lds) {
    for (int o = 32; o > 0; o >>= 1) merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) lds[2 * w] = m, lds[2 * w + 1] = s;
    __syncthreads();
    m = lds[0], s = lds[1];
    for (int i = 1; i < NT / 64; ++i) merge(m, s, lds[2 * i], lds[2 * i + 1]);
}

template <int NT>
__device__ float block_sum(float v, float* lds) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) lds[w] = v;
    __syncthreads();
    float r = lds[0];
    for (int i = 1; i < NT / 64; ++i) r += lds[i];
    return r;
}

// One workgroup per row pair.  VEC: rows start on 16-byte boundaries.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void accept_rate_rows(int64_t V, const T* __restrict__ d, int64_t ldd,
                                                             const T* __restrict__ t, int64_t ldt,
                                                             float* __restrict__ out) {
    __shared__ float lds[2 * kThreads / 64];
    const int64_t n = blockIdx.x;
    const T* dr = d + n * ldd;
    const T* tr = t + n * ldt;
    constexpr int E = Vec<T>::N;
    const int64_t nvec = VEC ? V / E : 0;
    const int tid = threadIdx.x;

    float md = -INFINITY, sd = 0.f, mt = -INFINITY, st = 0.f;
    for (int64_t i = tid; i < nvec; i += kThreads) {
        float xd[E], xt[E];
        Vec<T>::load(dr, i * E, xd);
        Vec<T>::load(tr, i * E, xt);
        fold<E>(md, sd, xd);
        fold<E>(mt, st, xt);
    }
    for (int64_t v = nvec * E + tid; v < V; v += kThreads) {
        float xd[1] = {load_elem(dr, v)}, xt[1] = {load_elem(tr, v)};
        fold<1>(md, sd, xd);
        fold<1>(mt, st, xt);
    }
    block_merge<kThreads>(md, sd, lds);
    block_merge<kThreads>(mt, st, lds);

    const float mdl = md * kLog2e, mtl = mt * kLog2e;
    const float isd = 1.f / sd, ist = 1.f / st;
    float acc = 0.f;
    for (int64_t i = tid; i < nvec; i += kThreads) {
        float xd[E], xt[E];
        Vec<T>::load(dr, i * E, xd);
        Vec<T>::load(tr, i * E, xt);
#pragma unroll
        for (int e = 0; e < E; ++e) acc += fabsf(exp_shifted(xd[e], mdl) * isd - exp_shifted(xt[e], mtl) * ist);
    }
    for (int64_t v = nvec * E + tid; v < V; v += kThreads)
        acc += fabsf(exp_shifted(load_elem(dr, v), mdl) * isd - exp_shifted(load_elem(tr, v), mtl) * ist);
    acc = block_sum<kThreads>(acc, lds);
    if (tid == 0) out[n] = 1.f - 0.5f * acc;
}

template <typename T>
hipError_t launch_typed(int64_t N, int64_t V, const void* d, int64_t ldd, const void* t, int64_t ldt, float* out,
                        hipStream_t stream) {
    const bool vec = ((uintptr_t)d % 16 == 0) && ((uintptr_t)t % 16 == 0) && ((ldd * sizeof(T)) % 16 == 0) &&
                     ((ldt * sizeof(T)) % 16 == 0);
    const T* dp = static_cast<const T*>(d);
    const T* tp = static_cast<const T*>(t);
    for (int64_t n0 = 0; n0 < N; n0 += 0x7fffffff) {  // grid.x limit
        const int64_t cnt = (N - n0) < 0x7fffffff ? (N - n0) : 0x7fffffff;
        if (vec)
            hipLaunchKernelGGL((accept_rate_rows<T, true>), dim3((uint32_t)cnt), dim3(kThreads), 0, stream, V,
                               dp + n0 * ldd, ldd, tp + n0 * ldt, ldt, out + n0);
        else
            hipLaunchKernelGGL((accept_rate_rows<T, false>), dim3((uint32_t)cnt), dim3(kThreads), 0, stream, V,
                               dp + n0 * ldd, ldd, tp + n0 * ldt, ldt, out + n0);
    }
    return hipGetLastError();
}

}  // namespace

size_t accept_rate_workspace(int64_t, int64_t) { return 0; }

hipError_t accept_rate_launch(int64_t N, int64_t V, int dtype, const void* d, int64_t ldd, const void* t,
                              int64_t ldt, float* out, void*, hipStream_t stream) {
    if (dtype == kBF16) return launch_typed<bf16_t>(N, V, d, ldd, t, ldt, out, stream);
    return launch_typed<float>(N, V, d, ldd, t, ldt, out, stream);
}

}  // namespace dspark
