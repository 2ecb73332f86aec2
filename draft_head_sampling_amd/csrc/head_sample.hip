// Sequential Markov-head block sampler with the confidence head and survival
// products ("基于 DSpark 的投机解码训练框架原理与实现", wangjunjian.com:
// section 3.2, paper eq. 5 and the block sampling loop; section 3.3, the
// confidence head and Algorithm 1's survival products; dpshk.com article on
// the Qwen3.8-27B-DSpark confidence head, section 2).
//
// One block of gamma positions is sampled per request.  Step k needs the
// token chosen at step k-1 by a vocabulary-wide argmax, so the steps form a
// chain of grid-wide dependencies:
//   init    zero the per-step argmax keys; hidden part of every confidence
//           logit, w_h . h[b,k] (it does not depend on sampled tokens)
//   step k  gather e = W1[x_{k-1}] into LDS, stream a tile of W2 rows,
//           bias[v] = W2[v] . e with fp32 accumulation (a short dot per row,
//           reduced across the lanes that share the row), z = U + bias (+ G),
//           tile argmax, one packed 64-bit atomicMax per request
//   finish decode tokens, add the Markov part of the confidence logit,
//           sigmoid, running survival product
// The [B x V] bias never reaches HBM unless the caller asks for it.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;  // vocabulary rows per workgroup

// Previous token of request b at step k (0-based), or -1 once the request
// has hit an invalid token id.
__device__ __forceinline__ int32_t prev_token(int64_t b, int k, int64_t B, int64_t gamma, int64_t V,
                                              const int32_t* x0, const int32_t* force, const uint64_t* keys) {
    int64_t x;
    if (k == 0) {
        x = x0[b];
    } else {
        const uint64_t key = keys[(int64_t)(k - 1) * B + b];
        if (key == 0) return -1;
        const int32_t f = force ? force[b * gamma + k - 1] : -1;
        x = f >= 0 ? f : key_token(key);
    }
    return (x >= 0 && x < V) ? (int32_t)x : -1;
}

template <typename T>
struct Chunk;  // 16 bytes of a W2 row
template <>
struct Chunk<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, float (&x)[4]) {
        float4 r = *reinterpret_cast<const float4*>(p);
        x[0] = r.x, x[1] = r.y, x[2] = r.z, x[3] = r.w;
    }
};
template <>
struct Chunk<bf16_t> {
    static constexpr int N = 8;
    __device__ static void load(const bf16_t* p, float (&x)[8]) {
        uint4 r = *reinterpret_cast<const uint4*>(p);
        x[0] = widen_lo(r.x), x[1] = widen_hi(r.x), x[2] = widen_lo(r.y), x[3] = widen_hi(r.y);
        x[4] = widen_lo(r.z), x[5] = widen_hi(r.z), x[6] = widen_lo(r.w), x[7] = widen_hi(r.w);
    }
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
    uint32_t lo = __shfl_xor((uint32_t)v, o), hi = __shfl_xor((uint32_t)(v >> 32), o);
    return ((uint64_t)hi << 32) | lo;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sample_init(int64_t B, int64_t gamma, int64_t H, const T* __restrict__ h,
                                                        const T* __restrict__ w_conf, uint64_t* __restrict__ keys,
                                                        float* __restrict__ hdot) {
    __shared__ float red[kThreads / 64];
    const int64_t bk = blockIdx.x;  // b * gamma + k
    const int64_t b = bk / gamma, k = bk % gamma;
    if (threadIdx.x == 0) keys[k * B + b] = 0;
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < H; i += kThreads) s += load_elem(w_conf, i) * load_elem(h, bk * H + i);
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int i = 0; i < kThreads / 64; ++i) t += red[i];
        hdot[bk] = t;
    }
}

// LPR = lanes sharing one W2 row (16 bytes each); LPR == 0: any r, one row
// per thread with scalar loads.
template <typename T, int BG, int LPR>
__global__ __launch_bounds__(kThreads) void sample_step(int64_t B, int64_t gamma, int k, int64_t V, int64_t r,
                                                        const T* __restrict__ U, const T* __restrict__ W1,
                                                        const T* __restrict__ W2, const float* __restrict__ G,
                                                        const int32_t* __restrict__ x0,
                                                        const int32_t* __restrict__ force, uint64_t* keys,
                                                        float* __restrict__ logits_out, float* __restrict__ bias_out) {
    extern __shared__ float e_lds[];  // [BG][r]
    __shared__ float bias_lds[BG][kTile];
    __shared__ int32_t xprev[BG];
    __shared__ uint64_t red[BG][kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b0 = (int64_t)blockIdx.y * BG;
    const int64_t v0 = (int64_t)blockIdx.x * kTile;

    if (tid < BG) xprev[tid] = (b0 + tid < B) ? prev_token(b0 + tid, k, B, gamma, V, x0, force, keys) : -1;
    __syncthreads();
    for (int64_t i = tid; i < BG * r; i += kThreads) {
        const int32_t x = xprev[i / r];
        e_lds[i] = x >= 0 ? load_elem(W1, (int64_t)x * r + i % r) : 0.f;
    }
    __syncthreads();

    if constexpr (LPR > 0) {
        constexpr int E = Chunk<T>::N;
        constexpr int RPW = 64 / LPR;  // rows per wave per load
        const int c = lane % LPR;
        float ereg[BG][E];
#pragma unroll
        for (int bb = 0; bb < BG; ++bb)
#pragma unroll
            for (int i = 0; i < E; ++i) ereg[bb][i] = e_lds[bb * r + c * E + i];
#pragma unroll 4
        for (int rr = wave * RPW + lane / LPR; rr < kTile; rr += (kThreads / 64) * RPW) {
            const int64_t v = v0 + rr;
            float acc[BG];
#pragma unroll
            for (int bb = 0; bb < BG; ++bb) acc[bb] = 0.f;
            if (v < V) {
                float w[E];
                Chunk<T>::load(W2 + v * r + c * E, w);
#pragma unroll
                for (int bb = 0; bb < BG; ++bb)
#pragma unroll
                    for (int i = 0; i < E; ++i) acc[bb] = __builtin_fmaf(w[i], ereg[bb][i], acc[bb]);
            }
#pragma unroll
            for (int o = LPR / 2; o > 0; o >>= 1)
#pragma unroll
                for (int bb = 0; bb < BG; ++bb) acc[bb] += __shfl_xor(acc[bb], o);
            if (c == 0)
#pragma unroll
                for (int bb = 0; bb < BG; ++bb) bias_lds[bb][rr] = acc[bb];
        }
    } else {
        for (int rr = tid; rr < kTile; rr += kThreads) {
            const int64_t v = v0 + rr;
            float acc[BG];
            for (int bb = 0; bb < BG; ++bb) acc[bb] = 0.f;
            if (v < V)
                for (int64_t j = 0; j < r; ++j) {
                    const float w = load_elem(W2, v * r + j);
                    for (int bb = 0; bb < BG; ++bb) acc[bb] = __builtin_fmaf(w, e_lds[bb * r + j], acc[bb]);
                }
            for (int bb = 0; bb < BG; ++bb) bias_lds[bb][rr] = acc[bb];
        }
    }
    __syncthreads();

    uint64_t key[BG];
#pragma unroll
    for (int bb = 0; bb < BG; ++bb) {
        key[bb] = 0;
        const int64_t b = b0 + bb;
        for (int rr = tid; rr < kTile; rr += kThreads) {
            const int64_t v = v0 + rr;
            if (b < B && xprev[bb] >= 0 && v < V) {
                const int64_t o = (b * gamma + k) * V + v;
                const float bias = bias_lds[bb][rr];
                const float lg = load_elem(U, o) + bias;
                const float sc = G ? lg + G[o] : lg;
                if (bias_out) bias_out[o] = bias;
                if (logits_out) logits_out[o] = lg;
                key[bb] = umax64(key[bb], argmax_key(sc, (uint32_t)v));
            }
        }
        for (int o = 32; o > 0; o >>= 1) key[bb] = umax64(key[bb], shfl_xor_u64(key[bb], o));
        if (lane == 0) red[bb][wave] = key[bb];
    }
    __syncthreads();
    if (tid < BG && b0 + tid < B && xprev[tid] >= 0) {
        uint64_t m = red[tid][0];
        for (int i = 1; i < kThreads / 64; ++i) m = umax64(m, red[tid][i]);
        atomicMax((unsigned long long*)&keys[(int64_t)k * B + b0 + tid], (unsigned long long)m);
    }
}

template <typename T>
__global__ __launch_bounds__(64) void sample_finish(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                                    const T* __restrict__ W1, const T* __restrict__ w_conf,
                                                    float b_conf, const int32_t* __restrict__ x0,
                                                    const int32_t* __restrict__ force, const uint64_t* keys,
                                                    const float* __restrict__ hdot, int32_t* __restrict__ tokens,
                                                    float* __restrict__ conf, float* __restrict__ survival) {
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    float A = 1.f;
    for (int k = 0; k < gamma; ++k) {
        const int32_t x = prev_token(b, k, B, gamma, V, x0, force, keys);
        float s = 0.f;
        if (x >= 0)
            for (int64_t j = lane; j < r; j += 64) s += load_elem(w_conf, H + j) * load_elem(W1, (int64_t)x * r + j);
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        const float z = hdot[b * gamma + k] + s + b_conf;
        const float c = x >= 0 ? 1.f / (1.f + expf(-z)) : __builtin_nanf("");
        A = A * c;
        if (lane == 0) {
            tokens[b * gamma + k] = x >= 0 ? key_token(keys[(int64_t)k * B + b]) : -1;
            conf[b * gamma + k] = c;
            survival[b * gamma + k] = A;
        }
    }
}

struct Buffers {
    uint64_t* keys;
    float* hdot;
};

Buffers carve(void* ws, int64_t B, int64_t gamma) {
    char* p = static_cast<char*>(ws);
    Buffers s;
    s.keys = reinterpret_cast<uint64_t*>(p);
    p += ((size_t)(8 * B * gamma) + 255) / 256 * 256;
    s.hdot = reinterpret_cast<float*>(p);
    return s;
}

template <typename T, int BG>
hipError_t launch_steps(int lpr, int64_t B, int64_t gamma, int k, int64_t V, int64_t r, const T* U, const T* W1,
                        const T* W2, const float* G, const int32_t* x0, const int32_t* force, uint64_t* keys,
                        float* lo, float* bo, hipStream_t stream) {
    const dim3 grid((uint32_t)((V + kTile - 1) / kTile), (uint32_t)((B + BG - 1) / BG));
    const size_t shm = sizeof(float) * BG * r;
#define DSPARK_STEP(L)                                                                                           \
    hipLaunchKernelGGL((sample_step<T, BG, L>), grid, dim3(kThreads), shm, stream, B, gamma, k, V, r, U, W1, W2, \
                       G, x0, force, keys, lo, bo)
    switch (lpr) {
        case 1: DSPARK_STEP(1); break;
        case 2: DSPARK_STEP(2); break;
        case 4: DSPARK_STEP(4); break;
        case 8: DSPARK_STEP(8); break;
        case 16: DSPARK_STEP(16); break;
        case 32: DSPARK_STEP(32); break;
        case 64: DSPARK_STEP(64); break;
        default: DSPARK_STEP(0); break;
    }
#undef DSPARK_STEP
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, const void* U, const void* h,
                        const void* W1, const void* W2, const void* w_conf, float b_conf, const int32_t* x0,
                        const float* G, const int32_t* force, int32_t* tokens, float* conf, float* survival,
                        float* lo, float* bo, void* ws, hipStream_t stream) {
    const T* Ut = static_cast<const T*>(U);
    const T* W1t = static_cast<const T*>(W1);
    const T* W2t = static_cast<const T*>(W2);
    const T* wt = static_cast<const T*>(w_conf);
    Buffers s = carve(ws, B, gamma);

    hipLaunchKernelGGL((sample_init<T>), dim3((uint32_t)(B * gamma)), dim3(kThreads), 0, stream, B, gamma, H,
                       static_cast<const T*>(h), wt, s.keys, s.hdot);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    // lanes per W2 row: 16-byte chunks per row when rows are 16-byte aligned
    const int64_t row_bytes = r * (int64_t)sizeof(T);
    int lpr = 0;
    if (row_bytes % 16 == 0 && row_bytes / 16 <= 64 && (((uintptr_t)W2) % 16 == 0)) {
        const int64_t q = row_bytes / 16;
        if ((q & (q - 1)) == 0) lpr = (int)q;
    }
    for (int k = 0; k < gamma; ++k) {
        if (B == 1)
            err = launch_steps<T, 1>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, stream);
        else if (B == 2)
            err = launch_steps<T, 2>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, stream);
        else if (B <= 4)
            err = launch_steps<T, 4>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, stream);
        else
            err = launch_steps<T, 8>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, stream);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((sample_finish<T>), dim3((uint32_t)B), dim3(64), 0, stream, B, gamma, V, H, r, W1t, wt, b_conf,
                       x0, force, s.keys, s.hdot, tokens, conf, survival);
    return hipGetLastError();
}

}  // namespace

size_t head_sample_workspace(int64_t B, int64_t gamma, int64_t, int64_t) {
    return ((size_t)(8 * B * gamma) + 255) / 256 * 256 + ((size_t)(4 * B * gamma) + 255) / 256 * 256;
}

hipError_t head_sample_launch(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int dtype, const void* U,
                              const void* h, const void* W1, const void* W2, const void* w_conf, float b_conf,
                              const int32_t* x0, const float* gumbel, const int32_t* force, int32_t* tokens,
                              float* conf, float* survival, float* logits_out, float* bias_out, void* ws,
                              hipStream_t stream) {
    if (dtype == kBF16)
        return launch_typed<bf16_t>(B, gamma, V, H, r, U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, tokens,
                                    conf, survival, logits_out, bias_out, ws, stream);
    return launch_typed<float>(B, gamma, V, H, r, U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, tokens, conf,
                               survival, logits_out, bias_out, ws, stream);
}

}  // namespace dspark
