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
#include <type_traits>

#include "internal.h"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;  // vocabulary rows per workgroup

// Argmax key of request b at step k: the maximum over the ncopy key copies
// (layout [ncopy][gamma][B], one key per 128-byte line; copies and spacing
// spread the cross-workgroup atomics over many lines).
constexpr int kKeyStride = 16;  // u64 words between argmax keys: one 128-byte line each

__device__ __forceinline__ uint64_t* key_at(uint64_t* keys, int c, int64_t gamma, int64_t B, int k, int64_t b) {
    return keys + (((int64_t)c * gamma + k) * B + b) * kKeyStride;
}
__device__ __forceinline__ uint64_t step_key(const uint64_t* keys, int ncopy, int64_t gamma, int64_t B, int k,
                                             int64_t b) {
    uint64_t m = 0;
    for (int c = 0; c < ncopy; ++c) m = umax64(m, keys[(((int64_t)c * gamma + k) * B + b) * kKeyStride]);
    return m;
}

// Previous token of request b at step k (0-based), or -1 once the request
// has hit an invalid token id.
__device__ __forceinline__ int32_t prev_token(int64_t b, int k, int64_t B, int64_t gamma, int64_t V,
                                              const int32_t* x0, const int32_t* force, const uint64_t* keys,
                                              int ncopy = 1) {
    int64_t x;
    if (k == 0) {
        x = x0[b];
    } else {
        const uint64_t key = step_key(keys, ncopy, gamma, B, k - 1, b);
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

// step_key and prev_token over a whole wave (every lane calls, every lane
// gets the result): lane c reads key copy c, so the copies cost one round
// trip instead of one each.
__device__ __forceinline__ uint64_t wave_step_key(const uint64_t* keys, int ncopy, int64_t gamma, int64_t B, int k,
                                                  int64_t b, int lane) {
    uint64_t m = 0;
    for (int c = lane; c < ncopy; c += 64) m = umax64(m, keys[(((int64_t)c * gamma + k) * B + b) * kKeyStride]);
    for (int o = 32; o > 0; o >>= 1) m = umax64(m, shfl_xor_u64(m, o));
    return m;
}
__device__ __forceinline__ int32_t wave_prev_token(int64_t b, int k, int64_t B, int64_t gamma, int64_t V,
                                                   const int32_t* x0, const int32_t* force, const uint64_t* keys,
                                                   int ncopy, int lane) {
    int64_t x;
    if (k == 0) {
        x = x0[b];
    } else {
        const uint64_t key = wave_step_key(keys, ncopy, gamma, B, k - 1, b, lane);
        if (key == 0) return -1;
        const int32_t f = force ? force[b * gamma + k - 1] : -1;
        x = f >= 0 ? f : key_token(key);
    }
    return (x >= 0 && x < V) ? (int32_t)x : -1;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sample_init(int64_t B, int64_t gamma, int64_t H, const T* __restrict__ h,
                                                        const T* __restrict__ w_conf, uint64_t* __restrict__ keys,
                                                        int ncopy, float* __restrict__ hdot) {
    __shared__ float red[kThreads / 64];
    const int64_t bk = blockIdx.x;  // b * gamma + k
    const int64_t b = bk / gamma, k = bk % gamma;
    if (threadIdx.x < ncopy) *key_at(keys, threadIdx.x, gamma, B, (int)k, b) = 0;
    float s = 0.f;
    constexpr int E = Chunk<T>::N;  // 16-byte loads where rows allow
    const T* hr = h + bk * H;
    if (H % E == 0 && (uintptr_t)w_conf % 16 == 0 && (uintptr_t)hr % 16 == 0) {
        for (int64_t i = (int64_t)threadIdx.x * E; i < H; i += (int64_t)kThreads * E) {
            float x[E], y[E];
            Chunk<T>::load(w_conf + i, x);
            Chunk<T>::load(hr + i, y);
#pragma unroll
            for (int q = 0; q < E; ++q) s = __builtin_fmaf(x[q], y[q], s);
        }
    } else {
        for (int64_t i = threadIdx.x; i < H; i += kThreads) s += load_elem(w_conf, i) * load_elem(hr, i);
    }
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
                                                        float* __restrict__ logits_out, float* __restrict__ bias_out,
                                                        const float* __restrict__ eg) {
    extern __shared__ float e_lds[];  // [BG][r]
    __shared__ float bias_lds[BG][kTile];
    __shared__ int32_t xprev[BG];
    __shared__ uint64_t red[BG][kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b0 = (int64_t)blockIdx.y * BG;
    const int64_t v0 = (int64_t)blockIdx.x * kTile;

    if (tid < BG) xprev[tid] = (b0 + tid < B) ? prev_token(b0 + tid, k, B, gamma, V, x0, force, keys) : -1;
    __syncthreads();
    for (int64_t i = tid; i < BG * r; i += kThreads) {  // e = W1[x_prev], or the gated embedding
        const int32_t x = xprev[i / r];
        e_lds[i] = x < 0 ? 0.f : eg ? eg[(b0 + i / r) * r + i % r] : load_elem(W1, (int64_t)x * r + i % r);
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
        atomicMax((unsigned long long*)key_at(keys, 0, gamma, B, k, b0 + tid), (unsigned long long)m);
    }
}

// One workgroup per request, one wave per step (gamma <= 16): every step's
// confidence in parallel, then the running survival product.
constexpr int kFinishMaxGamma = 16;

template <typename T>
__global__ __launch_bounds__(64 * kFinishMaxGamma) void sample_finish(
    int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, const T* __restrict__ W1, const T* __restrict__ w_conf,
    float b_conf, const int32_t* __restrict__ x0, const int32_t* __restrict__ force, const uint64_t* keys, int ncopy,
    const float* __restrict__ hdot, int32_t* __restrict__ tokens, float* __restrict__ conf,
    float* __restrict__ survival) {
    __shared__ float cs[kFinishMaxGamma];
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    for (int k0 = 0; k0 < gamma; k0 += kFinishMaxGamma) {  // gamma beyond 16 takes several rounds
        const int k = k0 + (int)(threadIdx.x >> 6);
        if (k < gamma) {
            const int32_t x = wave_prev_token(b, k, B, gamma, V, x0, force, keys, ncopy, lane);
            const uint64_t key = wave_step_key(keys, ncopy, gamma, B, k, b, lane);
            float s = 0.f;
            if (x >= 0)
                for (int64_t j = lane; j < r; j += 64)
                    s += load_elem(w_conf, H + j) * load_elem(W1, (int64_t)x * r + j);
            for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
            const float z = hdot[b * gamma + k] + s + b_conf;
            const float c = x >= 0 ? 1.f / (1.f + expf(-z)) : __builtin_nanf("");
            if (lane == 0) {
                tokens[b * gamma + k] = x >= 0 ? key_token(key) : -1;
                conf[b * gamma + k] = c;
                cs[k - k0] = c;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float A = k0 == 0 ? 1.f : survival[b * gamma + k0 - 1];
            for (int kk = k0; kk < gamma && kk < k0 + kFinishMaxGamma; ++kk) {
                A = A * cs[kk - k0];
                survival[b * gamma + kk] = A;
            }
        }
        __syncthreads();
    }
    // this request's keys and hidden dots are read: the workspace goes back to zero
    uint64_t* kw = const_cast<uint64_t*>(keys);
    float* hw = const_cast<float*>(hdot);
    for (int64_t i = threadIdx.x; i < (int64_t)ncopy * gamma; i += blockDim.x)
        kw[(((i / gamma) * gamma + i % gamma) * B + b) * kKeyStride] = 0;
    for (int64_t i = threadIdx.x; i < gamma; i += blockDim.x) hw[b * gamma + i] = 0.f;
}

// Zero n words (the gated head's scratch, once the block is done).
__global__ __launch_bounds__(kThreads) void clear_words(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Gated Markov head ("基于 DSpark 的投机解码训练框架原理与实现", wangjunjian.com,
// section 3.2, GatedMarkovHead): the previous token's embedding e = W1[x_{k-1}]
// is gated before the projection, e' = sigmoid(Wg [h_k; e]) * e (elementwise,
// Wg [r][H + r]), and the bias is W2 . e'.  The pages leave the map back to
// the vocabulary open; this is the vanilla head's W2.  The confidence head
// still sees e.  The hidden half of the gate, Wg[:, :H] . h_k, does not
// depend on sampled tokens and is computed once per call; the rest runs per
// step once the previous token is known.  Gated calls take the per-step
// path (on the matrix cores for bf16, r = 256, B >= 16).
// ---------------------------------------------------------------------------
// Dot product of n elements over the 64 lanes of a wave (every lane gets the
// sum); 16-byte loads when both rows are 16-byte aligned and n is a whole
// number of vectors.
template <typename T>
__device__ __forceinline__ float wave_dot(const T* __restrict__ a, const T* __restrict__ b, int64_t n, int lane) {
    constexpr int E = Chunk<T>::N;
    float s = 0.f;
    if (n % E == 0 && (uintptr_t)a % 16 == 0 && (uintptr_t)b % 16 == 0) {
        for (int64_t i = (int64_t)lane * E; i < n; i += 64 * E) {
            float x[E], y[E];
            Chunk<T>::load(a + i, x);
            Chunk<T>::load(b + i, y);
#pragma unroll
            for (int q = 0; q < E; ++q) s = __builtin_fmaf(x[q], y[q], s);
        }
    } else {
        for (int64_t i = lane; i < n; i += 64) s += load_elem(a, i) * load_elem(b, i);
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
}

constexpr int kGateRows = 16;  // gate rows per workgroup (4 per wave)

// grid (B * gamma, r / kGateRows): Ah[bk][j] = Wg[j, :H] . h[bk, :]
template <typename T>
__global__ __launch_bounds__(kThreads) void gate_hidden(int64_t H, int64_t r, const T* __restrict__ h,
                                                        const T* __restrict__ Wg, float* __restrict__ Ah) {
    const int64_t bk = blockIdx.x;  // b * gamma + k
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T* hr = h + bk * H;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    for (int64_t j = j0 + wave; j < j0 + kGateRows && j < r; j += kThreads / 64) {
        const float s = wave_dot(Wg + j * (H + r), hr, H, lane);
        if (lane == 0) Ah[bk * r + j] = s;
    }
}

// grid (B, r / kGateRows) at step k: e'[j] = sigmoid(Ah + Wg[j, H:] . e) * e[j].
template <typename T>
__global__ __launch_bounds__(kThreads) void gate_step(int64_t B, int64_t gamma, int k, int64_t V, int64_t H,
                                                      int64_t r, const T* __restrict__ W1, const T* __restrict__ Wg,
                                                      const int32_t* __restrict__ x0,
                                                      const int32_t* __restrict__ force, const uint64_t* keys,
                                                      int ncopy, const float* __restrict__ Ah,
                                                      float* __restrict__ eg) {
    __shared__ int32_t xs;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x < 64) {
        const int32_t x = wave_prev_token(b, k, B, gamma, V, x0, force, keys, ncopy, lane);
        if (lane == 0) xs = x;
    }
    __syncthreads();
    const int32_t x = xs;
    if (x < 0) return;  // the request stopped: its bias is never formed
    const T* e = W1 + (int64_t)x * r;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    for (int64_t j = j0 + wave; j < j0 + kGateRows && j < r; j += kThreads / 64) {
        const float s = wave_dot(Wg + j * (H + r) + H, e, r, lane);
        if (lane == 0) {
            const float z = Ah[(b * gamma + k) * r + j] + s;
            eg[b * r + j] = load_elem(e, j) / (1.f + expf(-z));
        }
    }
}

// 8-lane-chunk dot of two bf16 vectors held as 16-byte pieces, summed over the wave.
__device__ __forceinline__ float wave_dot8(uint4 a, uint4 b) {
    float s = 0.f;
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s = __builtin_fmaf(widen_lo(aw[q]), widen_lo(bw[q]), s);
        s = __builtin_fmaf(widen_hi(aw[q]), widen_hi(bw[q]), s);
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
}

constexpr int kGateRowsPerWave = kGateRows / (kThreads / 64);

// gate_step for bf16 with r <= 512, r % 8 == 0 and 16-byte aligned rows: lane
// l holds rank elements 8l .. 8l + 7.  The gate weights and the hidden halves
// do not depend on the previous token, so their loads are issued before it is
// known and overlap that round trip.
__global__ __launch_bounds__(kThreads) void gate_step_bf16(int64_t B, int64_t gamma, int k, int64_t V, int64_t H,
                                                           int64_t r, const bf16_t* __restrict__ W1,
                                                           const bf16_t* __restrict__ Wg,
                                                           const int32_t* __restrict__ x0,
                                                           const int32_t* __restrict__ force, const uint64_t* keys,
                                                           int ncopy, const float* __restrict__ Ah,
                                                           float* __restrict__ eg) {
    __shared__ int32_t xs;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    const bool mine = 8 * lane < r;
    uint4 wv[kGateRowsPerWave];
    float ah[kGateRowsPerWave];
#pragma unroll
    for (int i = 0; i < kGateRowsPerWave; ++i) {
        const int64_t j = j0 + wave + (kThreads / 64) * i;
        wv[i] = (j < r && mine) ? *reinterpret_cast<const uint4*>(Wg + j * (H + r) + H + 8 * lane) : uint4{0, 0, 0, 0};
        ah[i] = j < r ? Ah[(b * gamma + k) * r + j] : 0.f;
    }
    if (threadIdx.x < 64) {
        const int32_t x = wave_prev_token(b, k, B, gamma, V, x0, force, keys, ncopy, lane);
        if (lane == 0) xs = x;
    }
    __syncthreads();
    const int32_t x = xs;
    if (x < 0) return;  // the request stopped: its bias is never formed
    const bf16_t* e = W1 + (int64_t)x * r;
    const uint4 ev = mine ? *reinterpret_cast<const uint4*>(e + 8 * lane) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kGateRowsPerWave; ++i) {
        const int64_t j = j0 + wave + (kThreads / 64) * i;
        const float sdot = wave_dot8(wv[i], ev);
        if (lane == 0 && j < r) eg[b * r + j] = load_elem(e, j) / (1.f + expf(-(ah[i] + sdot)));
    }
}

// ---------------------------------------------------------------------------
// RNN head (the same page, section 3.2, RNNHead; paper eq. 6): a recurrent
// state replaces the embedding in the bias,
//   z = [s_{k-1}; e; h_k],  u = sigmoid(Wrg z),  s_k = u s_{k-1} + (1 - u) tanh(Wrc z)
// with s_0 = 0 and bias = W2 . s_k (Wrg, Wrc [r][2r + H]).  The h_k halves
// of both products are computed once per call; the rest per step.
// ---------------------------------------------------------------------------
// Dot of a row of T with a float vector over a wave (every lane gets the sum).
template <typename T>
__device__ __forceinline__ float wave_dot_f(const T* __restrict__ a, const float* __restrict__ b, int64_t n,
                                            int lane) {
    constexpr int E = Chunk<T>::N;
    float s = 0.f;
    if (n % E == 0 && (uintptr_t)a % 16 == 0) {
        for (int64_t i = (int64_t)lane * E; i < n; i += 64 * E) {
            float x[E];
            Chunk<T>::load(a + i, x);
#pragma unroll
            for (int q = 0; q < E; ++q) s = __builtin_fmaf(x[q], b[i + q], s);
        }
    } else {
        for (int64_t i = lane; i < n; i += 64) s += load_elem(a, i) * b[i];
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
}

// grid (B * gamma, r / kGateRows): Ag = Wrg[:, 2r:] . h_k and Ac = Wrc[:, 2r:] . h_k
template <typename T>
__global__ __launch_bounds__(kThreads) void rnn_hidden(int64_t H, int64_t r, const T* __restrict__ h,
                                                       const T* __restrict__ Wrg, const T* __restrict__ Wrc,
                                                       float* __restrict__ Ag, float* __restrict__ Ac) {
    const int64_t bk = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t Z = 2 * r + H;
    const T* hr = h + bk * H;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    for (int64_t j = j0 + wave; j < j0 + kGateRows && j < r; j += kThreads / 64) {
        const float g = wave_dot(Wrg + j * Z + 2 * r, hr, H, lane);
        const float c = wave_dot(Wrc + j * Z + 2 * r, hr, H, lane);
        if (lane == 0) Ag[bk * r + j] = g, Ac[bk * r + j] = c;
    }
}

// grid (B, r / kGateRows) at step k: the new state s_k of every request
// (written to s_out; s_in holds s_{k-1}, ignored at k = 0).
template <typename T>
__global__ __launch_bounds__(kThreads) void rnn_step(int64_t B, int64_t gamma, int k, int64_t V, int64_t H, int64_t r,
                                                     const T* __restrict__ W1, const T* __restrict__ Wrg,
                                                     const T* __restrict__ Wrc, const int32_t* __restrict__ x0,
                                                     const int32_t* __restrict__ force, const uint64_t* keys,
                                                     int ncopy, const float* __restrict__ Ag,
                                                     const float* __restrict__ Ac,
                                                     const float* __restrict__ s_in, float* __restrict__ s_out) {
    extern __shared__ float z_s[];  // [2r]: s_{k-1}, then e
    __shared__ int32_t xs;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x < 64) {
        const int32_t x = wave_prev_token(b, k, B, gamma, V, x0, force, keys, ncopy, lane);
        if (lane == 0) xs = x;
    }
    __syncthreads();
    const int32_t x = xs;
    if (x < 0) return;  // the request stopped: its bias is never formed
    for (int64_t i = threadIdx.x; i < r; i += kThreads) {
        z_s[i] = k == 0 ? 0.f : s_in[b * r + i];
        z_s[r + i] = load_elem(W1, (int64_t)x * r + i);
    }
    __syncthreads();
    const int64_t Z = 2 * r + H, bk = b * gamma + k;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    for (int64_t j = j0 + wave; j < j0 + kGateRows && j < r; j += kThreads / 64) {
        const float zg = Ag[bk * r + j] + wave_dot_f(Wrg + j * Z, z_s, 2 * r, lane);
        const float zc = Ac[bk * r + j] + wave_dot_f(Wrc + j * Z, z_s, 2 * r, lane);
        if (lane == 0) {
            const float u = 1.f / (1.f + expf(-zg));
            s_out[b * r + j] = u * z_s[j] + (1.f - u) * tanhf(zc);
        }
    }
}

// rnn_step for bf16 with r <= 256, r % 8 == 0 and 16-byte aligned rows: lane
// l holds elements 8l .. 8l + 7 of z's first 2r entries [s_{k-1}; e].  The
// weights, the hidden halves and s_{k-1} do not depend on the previous token,
// so their loads are issued before it is known.
__global__ __launch_bounds__(kThreads) void rnn_step_bf16(int64_t B, int64_t gamma, int k, int64_t V, int64_t H,
                                                          int64_t r, const bf16_t* __restrict__ W1,
                                                          const bf16_t* __restrict__ Wrg,
                                                          const bf16_t* __restrict__ Wrc,
                                                          const int32_t* __restrict__ x0,
                                                          const int32_t* __restrict__ force, const uint64_t* keys,
                                                          int ncopy, const float* __restrict__ Ag,
                                                          const float* __restrict__ Ac,
                                                          const float* __restrict__ s_in, float* __restrict__ s_out) {
    __shared__ int32_t xs;
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t Z = 2 * r + H, bk = b * gamma + k;
    const int64_t j0 = (int64_t)blockIdx.y * kGateRows;
    const int c0 = 8 * lane;  // first z element of this lane
    const bool sp = c0 < r, ep = !sp && c0 < 2 * r;  // state part, embedding part
    uint4 wg[kGateRowsPerWave], wc[kGateRowsPerWave];
    float ag[kGateRowsPerWave], ac[kGateRowsPerWave], sj[kGateRowsPerWave];
#pragma unroll
    for (int i = 0; i < kGateRowsPerWave; ++i) {
        const int64_t j = j0 + wave + (kThreads / 64) * i;
        const bool ok = j < r && (sp || ep);
        wg[i] = ok ? *reinterpret_cast<const uint4*>(Wrg + j * Z + c0) : uint4{0, 0, 0, 0};
        wc[i] = ok ? *reinterpret_cast<const uint4*>(Wrc + j * Z + c0) : uint4{0, 0, 0, 0};
        ag[i] = j < r ? Ag[bk * r + j] : 0.f;
        ac[i] = j < r ? Ac[bk * r + j] : 0.f;
        sj[i] = (j < r && k > 0) ? s_in[b * r + j] : 0.f;
    }
    float zs[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) zs[q] = 0.f;
    if (sp && k > 0) {
        const float4 a = *reinterpret_cast<const float4*>(s_in + b * r + c0);
        const float4 c = *reinterpret_cast<const float4*>(s_in + b * r + c0 + 4);
        zs[0] = a.x, zs[1] = a.y, zs[2] = a.z, zs[3] = a.w, zs[4] = c.x, zs[5] = c.y, zs[6] = c.z, zs[7] = c.w;
    }
    if (threadIdx.x < 64) {
        const int32_t x = wave_prev_token(b, k, B, gamma, V, x0, force, keys, ncopy, lane);
        if (lane == 0) xs = x;
    }
    __syncthreads();
    const int32_t x = xs;
    if (x < 0) return;  // the request stopped: its bias is never formed
    if (ep) {
        const uint4 e = *reinterpret_cast<const uint4*>(W1 + (int64_t)x * r + (c0 - r));
        const uint32_t ew[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) zs[2 * q] = widen_lo(ew[q]), zs[2 * q + 1] = widen_hi(ew[q]);
    }
#pragma unroll
    for (int i = 0; i < kGateRowsPerWave; ++i) {
        const int64_t j = j0 + wave + (kThreads / 64) * i;
        float g = 0.f, c = 0.f;
        const uint32_t gw[4] = {wg[i].x, wg[i].y, wg[i].z, wg[i].w}, cw[4] = {wc[i].x, wc[i].y, wc[i].z, wc[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g = __builtin_fmaf(widen_lo(gw[q]), zs[2 * q], g);
            g = __builtin_fmaf(widen_hi(gw[q]), zs[2 * q + 1], g);
            c = __builtin_fmaf(widen_lo(cw[q]), zs[2 * q], c);
            c = __builtin_fmaf(widen_hi(cw[q]), zs[2 * q + 1], c);
        }
        for (int o = 32; o > 0; o >>= 1) g += __shfl_xor(g, o), c += __shfl_xor(c, o);
        if (lane == 0 && j < r) {
            const float u = 1.f / (1.f + expf(-(ag[i] + g)));
            s_out[b * r + j] = u * sj[i] + (1.f - u) * tanhf(ac[i] + c);
        }
    }
}

// ---------------------------------------------------------------------------
// Single-request chain kernel (B = 1, bf16, rank 256).
//
// One persistent workgroup per CU owns a contiguous slice of the vocabulary
// and keeps its W2 rows in registers for the whole block, so W2 crosses HBM
// once per call instead of once per step.  A row is split over 8 lanes (32
// bf16 each); a step is 16 v_dot2c_f32_bf16 per held row slot plus a 3-level
// DPP reduction across the 8 lanes.  The grid-wide dependency between steps
// goes through one 128-byte slot per workgroup and step holding two 64-bit
// words: the workgroup's packed argmax key (never zero) and its partial sum
// of the confidence logit, w_h . h over a 1/nwg slice of the hidden state,
// tagged with a set bit 32 so it is never zero either.  Every workgroup polls
// all slots of the step until no word is zero, then takes the maximum key as
// the winner and sums the partials in slot order.  Each word is its own flag,
// so the exchange needs no counter and no fence; spacing the slots one
// 128-byte line apart spreads the polling over memory channels.  U and G of
// the next step are loaded before they are needed.  The last workgroup to
// leave zeroes the slots, so the workspace is ready for the next call.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// DPP lane permutations: quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1]
// (xor 2), row_half_mirror (lane i <- 7-i in each group of 8), row_mirror
// (lane i <- 15-i in each row of 16).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
// Sum over each aligned group of 8 lanes, result in all 8 lanes.
__device__ __forceinline__ float sum8(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    return v;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
// Maximum over the 64 lanes of a wave (wave-uniform result).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
    k = umax64(k, dpp_u64<kDppXor1>(k));
    k = umax64(k, dpp_u64<kDppXor2>(k));
    k = umax64(k, dpp_u64<kDppHalfMirror>(k));
    k = umax64(k, dpp_u64<kDppMirror>(k));
    return umax64(umax64(readlane_u64(k, 0), readlane_u64(k, 16)), umax64(readlane_u64(k, 32), readlane_u64(k, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

constexpr int kChainThreads = 512;  // 8 waves: 256 registers per lane hold the W2 slice
constexpr int kChainWaves = kChainThreads / 64;
constexpr int kChainLanesPerRow = 8;
constexpr int kChainGroups = kChainThreads / kChainLanesPerRow;  // rows per slot
constexpr int kChainRank = 256;
constexpr int kChainMaxSlots = 10;  // 160 registers of W2 per lane; more spills
constexpr int kChainMaxWGs = 256;   // 4 slots per lane when polling
constexpr int kSlotWords = 16;      // 128-byte stride between slots (key, partial logit, padding)
constexpr int kChainPoll = kChainMaxWGs / 64;
constexpr int kChainSpinLimit = 1 << 21;
constexpr size_t kChainHeader = kWsHeader;  // words 0 (exit counter), 1 (status), 3 (paths)

// Candidate screen.  The Markov bias of a row is bounded by Cauchy-Schwarz,
// |W2[v] . e| <= |W2[v]| |e|, so at step k only rows whose bias-free score
// t_v = U_k[v] (+ G_k[v]) lies within twice that bound (plus rounding
// slack) of the best t can win the argmax.  Every row workgroup publishes,
// per step, its three best rows by ranking key (the order-preserving image
// of t with the low 10 bits replaced by the row's index in the workgroup),
// the fourth key as a cutoff, a bound on |U| + |G| and its slice of the
// hidden part of the confidence logit.  Workgroup 0, which holds no rows,
// keeps the entries within a window of the best t (best t minus a guess of
// twice the bound), stages their W1 and W2 rows in LDS, precomputes every
// bias the chain can need and walks the chain in one wave, first with the
// guessed bound and, if the largest W2 row norm turns out larger, again.  The
// W2 rows stream through registers only for that norm, from the start but
// throttled: three waves per workgroup with one 64-byte row slice in flight
// per lane, so the stream ends about when the coordinator needs the norm
// while the lists and the coordinator's reads do not queue behind it (a
// full-rate stream makes every cross-workgroup message wait several
// microseconds).  A step whose candidate set is not provably inside the
// lists hands the rest of the block to the grid-wide per-step exchange,
// which then keeps each workgroup's W2 rows in registers.
constexpr int kScreenMaxGamma = 8;   // U and G of every step stay in registers during the screen
// A row workgroup's region: word k (k < kScreenMaxGamma) is the step-k
// summary, (best ranking key << 32) | (|U|+|G| bound bits | 1) (the low bit
// makes the word non-zero and the bound one ulp larger, still a bound), all
// in the region's first 64 bytes; then kScreenStep list words per step from
// kListBase (3 entries, cutoff); then the largest squared W2 row norm.
constexpr int kScreenStep = 4;       // list words per step: 3 entries, cutoff
constexpr int kScreenEntries = 3;
constexpr int kScreenWaves = kChainWaves / 2;  // row workgroups: waves that screen; the others take the norms
constexpr int kScreenLanes = 64 * kScreenWaves;
constexpr int kScreenRows = 3;       // rows per screening lane
constexpr int kNormWaves = 3;        // of the other waves, those that stream W2 for the norm
constexpr int kNormLanes = 64 * kNormWaves;
constexpr int kNormGroups = kNormLanes / kChainLanesPerRow;  // rows per norm slot
constexpr int kStreamSlots = 1;      // W2 row slices in flight per norm lane
constexpr int kRegionWords = 64;     // u64 words per workgroup region: one per lane of a wave
constexpr int kPollRegions = kChainMaxWGs / kChainWaves;  // regions polled per coordinator wave
constexpr int kCandMax = 32;         // candidate rows staged in LDS
constexpr int kCandPerWave = kCandMax / kChainWaves;
constexpr int kSampleRows = kChainThreads / kChainLanesPerRow;  // W2 rows sampled for the window guess
constexpr int kLidBits = 10;         // row index inside a workgroup (rows_per_wg <= 640)
constexpr uint32_t kLidMask = (1u << kLidBits) - 1;
constexpr uint64_t kEmptyEntry = 1ull << 31;         // no row (low word above any row id + 1)
constexpr uint64_t kTag = 1ull << 32;                // marks a written scalar word
constexpr uint64_t kDecideDone = 1ull << 63;
constexpr uint64_t kDecideResume = 1ull << 62;       // | step << 32 | previous token
// The word that every row workgroup polls (the decision) is replicated, one
// 128-byte line per copy, so the polls spread over memory channels;
// workgroup g reads copy g % kCopies.
constexpr int kCopies = 16;
constexpr int kAuxWords = kCopies * kSlotWords;
constexpr float kN2Guess = 1.5f;                     // sampled squared norm -> guess of the largest
constexpr int kListBase = kScreenMaxGamma;
constexpr int kNormWord = kListBase + kScreenStep * kScreenMaxGamma;
constexpr int kRegionUsed = kNormWord + 1;
static_assert(kRegionUsed <= kRegionWords, "screen region too small");
static_assert(kChainRank / 2 % 64 == 0, "16-byte aligned rows in LDS");
static_assert(kScreenMaxGamma == 8 && kPollRegions % 8 == 0, "one 64-byte summary line per region, 8 regions per load");
static_assert(kCandMax % kChainWaves == 0, "candidates per wave");
static_assert(kChainMaxSlots * kChainGroups <= (1 << kLidBits), "row index field too small");
static_assert(kChainMaxSlots * kChainGroups <= kScreenRows * kScreenLanes, "screening lanes cover the rows");
// Slack on the bias bound: covers fp32 rounding of the squared norms, of the
// square roots and of any summation order of a 256-term dot product
// (relative 256 * 2^-24 each), with a wide margin.
constexpr float kBetaSlack = 1.0f + 1.0f / 256;
constexpr float kBetaFloor = 1e-30f;  // products flushed as denormals
constexpr float kUlp = 0x1p-24f;

__device__ __forceinline__ void load64B(const bf16_t* p, uint32_t (&r)[16]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 t = q[i];
        r[4 * i] = t.x, r[4 * i + 1] = t.y, r[4 * i + 2] = t.z, r[4 * i + 3] = t.w;
    }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = __builtin_fmaxf(v, dpp_f32<kDppXor1>(v));
    v = __builtin_fmaxf(v, dpp_f32<kDppXor2>(v));
    v = __builtin_fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = __builtin_fmaxf(v, dpp_f32<kDppMirror>(v));
    return __builtin_fmaxf(__builtin_fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
                           __builtin_fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
}

// Ends of t over a 32-bit ranking key's bucket; key 0 (no row) is -infinity.
__device__ __forceinline__ double key_lower(uint32_t q) {
    return q == 0 ? -__builtin_inf() : (double)from_orderable(q & ~kLidMask);
}
__device__ __forceinline__ double key_upper(uint32_t q) {
    return q == 0 ? -__builtin_inf() : (double)from_orderable(q | kLidMask);
}
// Non-negative float bits with NaN and overflow mapped to +infinity, so an
// unsigned max over them is a float max that cannot lose a NaN.
__device__ __forceinline__ uint32_t bound_bits(float a) {
    return a <= 3.402823466e38f ? __float_as_uint(a) : 0x7f800000u;
}
__device__ __forceinline__ bool finite_bits(uint32_t b) { return b < 0x7f800000u; }
// Largest float not above x (NaN stays NaN).
__device__ __forceinline__ float float_down(double x) {
    float f = (float)x;
    if ((double)f > x) {  // one representable step down
        const uint32_t b = __float_as_uint(f);
        f = __uint_as_float(f > 0.f ? b - 1 : f < 0.f ? b + 1 : 0x80000001u);
    }
    return f;
}
__device__ __forceinline__ uint32_t ranking_key(float t, uint32_t lid) {
    return (orderable(t) & ~kLidMask) | lid;
}

constexpr int kERows = kCandMax + 1 + kScreenMaxGamma;  // e rows: candidates' W1 rows, anchor, forced
constexpr int kERowAnchor = kCandMax;
constexpr int kERowForced = kCandMax + 1;
static_assert(kERows <= 64, "one e row per lane");

struct __align__(16) ScreenLds {  // (16-byte rows: the bias table reads them as uint4)
    uint32_t cw2[kCandMax][kChainRank / 2];         // W2 rows of the candidates (bf16 pairs)
    uint32_t cw1[kCandMax][kChainRank / 2];         // their W1 rows: e of the next step if one wins
    float bias[kCandMax][kERows];                   // W2[candidate] . e for every possible predecessor
    uint32_t fw1[kScreenMaxGamma][kChainRank / 2];  // W1 rows of teacher-forced tokens
    uint32_t e0[kChainRank / 2];                    // W1 row of the anchor
    uint32_t cv[kCandMax];
    int cstep[kCandMax];
    float cu[kCandMax], cg[kCandMax], ct[kCandMax];
    float esq[kERows], zcm[kERows];                 // |e|^2 and w_e . e of every e row
    uint32_t stepmask[kScreenMaxGamma];             // candidates of each step
    float pw[kScreenMaxGamma][kChainWaves];
    uint32_t wn[kChainWaves];
    uint32_t kmax[kChainWaves][kScreenMaxGamma];  // per wave and step: best ranking key, |U|+|G| bound bits
    uint32_t bmax[kChainWaves][kScreenMaxGamma];
    uint32_t fkey[kScreenMaxGamma], fbound[kScreenMaxGamma];  // over all regions
    uint32_t fcut[kScreenMaxGamma];  // largest cutoff of the regions whose lists were read
    float pk[kScreenMaxGamma];
    float winf[kScreenMaxGamma];
    uint32_t wkey[kScreenMaxGamma];                 // the windows as ranking-key bounds
    // after e row r at step k: the e row of step k + 1 (-1: unproven, -2:
    // the step's token is out of range), and the step's sampled token
    int2 tjt[kScreenMaxGamma][kERows];
    uint32_t wtop[kScreenMaxGamma][kScreenWaves][4];  // row workgroup: each wave's best keys
    uint32_t a1[kScreenMaxGamma];
    int sync;                                        // arrivals of the screening waves
    int32_t fv[kScreenMaxGamma];
    int overflow[kScreenMaxGamma];
    uint32_t n2, n2s;
    int ncand, abort;
    uint64_t decision;
};

// Hidden part of the confidence logit of every step over this workgroup's
// slice [h_lo, h_hi) of H, from `nt` threads: per-thread sums over chunks
// of nt elements, then fixed-order wave sums into s.pw[k][wave].  The loads
// of a chunk are unconditional from clamped indices (a load under a branch
// would be waited for at the branch's end, one round trip per load).
__device__ __forceinline__ void hidden_partials(ScreenLds& s, int gamma, int64_t H, int64_t h_lo, int64_t h_hi,
                                                const bf16_t* __restrict__ h, const bf16_t* __restrict__ w_conf,
                                                int t, int nt, int lane, int wave) {
    float p[kScreenMaxGamma];
#pragma unroll
    for (int k = 0; k < kScreenMaxGamma; ++k) p[k] = 0.f;
    // 16-byte pieces, two per thread, all loads of a round in flight together
    // (so cold data costs one memory latency per round, not one per element
    // group); other shapes take the element loop below
    const bool vec = (h_lo & 7) == 0 && ((h_hi - h_lo) & 7) == 0 && (H & 7) == 0 &&
                     (((uintptr_t)h | (uintptr_t)w_conf) & 15) == 0;
    constexpr int kPieces = 2;
    for (int64_t base = h_lo; vec && base < h_hi; base += (int64_t)8 * nt * kPieces) {  // workgroup-uniform
        uint4 wv[kPieces], hv[kPieces][kScreenMaxGamma];
        bool use[kPieces];
#pragma unroll
        for (int pc = 0; pc < kPieces; ++pc) {
            const int64_t i = base + 8 * (t + (int64_t)nt * pc);
            use[pc] = i < h_hi;
            const int64_t ic = use[pc] ? i : h_lo;
            wv[pc] = *reinterpret_cast<const uint4*>(w_conf + ic);
#pragma unroll
            for (int k = 0; k < kScreenMaxGamma; ++k)
                hv[pc][k] = *reinterpret_cast<const uint4*>(h + (int64_t)min(k, gamma - 1) * H + ic);
        }
#pragma unroll
        for (int pc = 0; pc < kPieces; ++pc) {
            if (!use[pc]) continue;
            const uint32_t ww[4] = {wv[pc].x, wv[pc].y, wv[pc].z, wv[pc].w};
#pragma unroll
            for (int k = 0; k < kScreenMaxGamma; ++k) {
                const uint32_t hw[4] = {hv[pc][k].x, hv[pc][k].y, hv[pc][k].z, hv[pc][k].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) p[k] = dot2(ww[e], hw[e], p[k]);
            }
        }
    }
    for (int64_t base = h_lo; !vec && base < h_hi; base += nt) {  // workgroup-uniform trip count
        const int64_t i = base + t;
        const bool use = i < h_hi;
        const int64_t ic = use ? i : 0;
        const uint16_t wb = w_conf[ic].bits;
        uint16_t hb[kScreenMaxGamma];
#pragma unroll
        for (int k = 0; k < kScreenMaxGamma; ++k) hb[k] = h[(int64_t)min(k, gamma - 1) * H + ic].bits;
        const float w = use ? __uint_as_float((uint32_t)wb << 16) : 0.f;
#pragma unroll
        for (int k = 0; k < kScreenMaxGamma; ++k) p[k] += w * __uint_as_float((uint32_t)hb[k] << 16);
    }
#pragma unroll
    for (int k = 0; k < kScreenMaxGamma; ++k) {
        if (k >= gamma) break;
        const float v = wave_sum_f32(p[k]);
        if (lane == 0) s.pw[k][wave] = v;
    }
}

// Barrier of the screening waves alone (the norm waves keep streaming): each
// wave's arrival is an LDS increment ordered after its earlier LDS writes.
__device__ __forceinline__ void screen_sync(ScreenLds& s, int lane, int target) {
    if (lane == 0) __hip_atomic_fetch_add(&s.sync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int spin = 0; spin < kChainSpinLimit; ++spin) {  // bounded like every wait here
        if (__hip_atomic_load(&s.sync, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int NSLOT>
__global__ __launch_bounds__(kChainThreads) void sample_chain_b1(
    int gamma, int64_t V, int64_t H, int rows_per_wg, int screen, const bf16_t* __restrict__ U,
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W2,
    const bf16_t* __restrict__ w_conf, float b_conf, const int32_t* __restrict__ x0, const float* __restrict__ G,
    const int32_t* __restrict__ force, int32_t* __restrict__ tokens, float* __restrict__ conf,
    float* __restrict__ survival, float* __restrict__ logits_out, float* __restrict__ bias_out, uint64_t* slots,
    uint64_t* regions, uint64_t* aux, uint32_t* header, int spin_limit, const uint32_t* __restrict__ nbound) {
    __shared__ uint64_t red[kChainWaves];
    __shared__ float fred[kChainWaves];
    __shared__ __align__(16) uint32_t we_lds[kChainRank / 2];  // Markov part of the confidence weights (workgroup 0)
    __shared__ uint64_t winner;
    __shared__ float zpart;
    __shared__ int last_flag;
    __shared__ ScreenLds sc;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = tid >> 3, sub = tid & 7;
    const int g = blockIdx.x, nwg = gridDim.x;
    const bool wg0 = g == 0;  // the coordinator: no vocabulary rows
    const int64_t row0 = wg0 ? V : (int64_t)(g - 1) * rows_per_wg;
    const int64_t h_per = (H + nwg - 1) / nwg;  // hidden elements of this workgroup's confidence partial
    const int64_t h_lo = (int64_t)g * h_per < H ? (int64_t)g * h_per : H;
    const int64_t h_hi = h_lo + h_per < H ? h_lo + h_per : H;
    uint64_t* const dcopy = aux + (g % kCopies) * kSlotWords;           // this workgroup's decision copy
    uint64_t* myregion = regions + (int64_t)g * kRegionWords;

    const int64_t xa = x0[0];
    const bool scr = screen && xa >= 0 && xa < V;  // the same in every workgroup
    // A weights-only bound from dspark_w2_bound, used when its fingerprint
    // names this W2 (address, vocabulary, rank): the largest squared row norm
    // and that of the rows the coordinator samples (checked below), in place
    // of the norm stream.  The same in every workgroup.
    bool bnd = false;
    uint32_t bnd_n2 = 0, bnd_n2s = 0;
    if (scr && nbound != nullptr) {
        uint32_t bw[kW2BoundWords];
#pragma unroll
        for (int i = 0; i < kW2BoundWords; ++i) bw[i] = nbound[i];
        bnd = bw[7] == kW2BoundTag && (((uint64_t)bw[3] << 32) | bw[2]) == (uint64_t)V && bw[4] == (uint32_t)kChainRank &&
              (((uint64_t)bw[6] << 32) | bw[5]) == (uint64_t)(uintptr_t)W2;
        bnd_n2 = bw[0];
        bnd_n2s = bw[1];
    }

    constexpr int NMINE = NSLOT > 8 ? 2 : 1;  // lane `sub` finishes slots sub and sub + 8
    int64_t my_v[NMINE];
    bool my_ok[NMINE];
#pragma unroll
    for (int m = 0; m < NMINE; ++m) {
        const int slot = sub + 8 * m;
        const int lr = slot * kChainGroups + grp;
        my_v[m] = row0 + lr;
        my_ok[m] = slot < NSLOT && lr < rows_per_wg && my_v[m] < V;
    }

    uint32_t w2[NSLOT][16];
    int k0 = 0;           // first step left to the grid-wide exchange
    int64_t x = xa;       // token before step k0
    bool valid = xa >= 0 && xa < V;
    bool done = false;    // the whole block is settled
    float A = 1.f;        // running survival (workgroup 0, thread 0)

    if (wg0) {
        if (tid < kChainRank / 2)
            we_lds[tid] = (uint32_t)w_conf[H + 2 * tid].bits | ((uint32_t)w_conf[H + 2 * tid + 1].bits << 16);
        if (scr) {
            // prologue: anchor row, forced tokens, own hidden slice, and a
            // sample of W2 rows whose largest norm sets the window guess
            uint32_t smp[16];
            load64B(W2 + (int64_t)grp * (V / kSampleRows) * kChainRank + sub * 32, smp);
            if (tid < kChainRank / 2) sc.e0[tid] = reinterpret_cast<const uint32_t*>(W1 + xa * kChainRank)[tid];
            if (tid < kScreenMaxGamma) {
                sc.fv[tid] = (force && tid < gamma) ? force[tid] : -1;
                sc.overflow[tid] = 0;
            }
            if (tid == 0) sc.ncand = 0, sc.abort = 0, sc.n2 = 0;
            // the whole hidden part of every confidence logit: the lists
            // arrive several microseconds after this is done
            hidden_partials(sc, gamma, H, 0, H, h, w_conf, tid, kChainThreads, lane, wave);
            {
                float a = 0.f;
#pragma unroll
                for (int q = 0; q < 16; ++q) a = dot2(smp[q], smp[q], a);
                const uint32_t m = wave_max_u32(bound_bits(sum8(a)));
                if (lane == 0) sc.wn[wave] = m;
            }
            __syncthreads();
            if (tid < gamma) {
                float ps = 0.f;
#pragma unroll
                for (int w = 0; w < kChainWaves; ++w) ps += sc.pw[tid][w];
                sc.pk[tid] = ps;
            }
            if (tid == kChainThreads - 1) {
                uint32_t m = 0;
#pragma unroll
                for (int w = 0; w < kChainWaves; ++w) m = max(m, sc.wn[w]);
                sc.n2s = m;
            }
            if (wave == 0) {
                const float es = wave_sum_f32(dot2(sc.e0[2 * lane + 1], sc.e0[2 * lane + 1],
                                                   dot2(sc.e0[2 * lane], sc.e0[2 * lane], 0.f)));
                if (lane == 0) sc.esq[kERowAnchor] = es;
            }

            // the summaries: wave w polls row workgroups 1 + w + 8 j (j < 32),
            // eight per load: lane l reads step l % 8 of workgroup
            // j = 8 q + l / 8 of load q; the spin only checks that every word
            // is written
            constexpr int kSumLoads = kPollRegions / 8;
            const int sk = lane & 7;
            uint64_t sw[kSumLoads];
            bool suse[kSumLoads];
            int sgg[kSumLoads];
#pragma unroll
            for (int q = 0; q < kSumLoads; ++q) {
                sgg[q] = 1 + wave + kChainWaves * (8 * q + (lane >> 3));
                suse[q] = sgg[q] < nwg && sk < gamma;
            }
            bool ready = false;
            for (int spin = 0; spin < spin_limit && !ready; ++spin) {
                bool all = true;
#pragma unroll
                for (int q = 0; q < kSumLoads; ++q) {
                    sw[q] = __hip_atomic_load(regions + (suse[q] ? (int64_t)sgg[q] * kRegionWords + sk : 0),
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    all = all && (!suse[q] || sw[q] != 0);
                }
                ready = __all(all);
                if (!ready) __builtin_amdgcn_s_sleep(1);
            }
            if (!ready && lane == 0) sc.abort = 1;
            {
                uint32_t km = 0, bm = 0;
#pragma unroll
                for (int q = 0; q < kSumLoads; ++q) {
                    km = suse[q] ? max(km, (uint32_t)(sw[q] >> 32)) : km;
                    bm = suse[q] ? max(bm, (uint32_t)sw[q]) : bm;
                }
                // lanes of one step: l, l ^ 8, l ^ 16, ...
#pragma unroll
                for (int o = 8; o < 64; o <<= 1) km = max(km, (uint32_t)__shfl_xor(km, o)), bm = max(bm, (uint32_t)__shfl_xor(bm, o));
                if (lane < kScreenMaxGamma) sc.kmax[wave][lane] = km, sc.bmax[wave][lane] = bm;
            }
            __syncthreads();
            if (tid < kScreenMaxGamma) {
                uint32_t km = 0, bm = 0;
#pragma unroll
                for (int w = 0; w < kChainWaves; ++w) km = max(km, sc.kmax[w][tid]), bm = max(bm, sc.bmax[w][tid]);
                sc.fkey[tid] = km;
                sc.fbound[tid] = bm;
                sc.fcut[tid] = 0;
            }
            __syncthreads();
            // the windows: best t minus twice a guess of the bias bound (the
            // sampled norm and the anchor row's norm, both enlarged) plus
            // rounding slack; the walk checks them against the real bound
            if (tid < gamma) {
                const float bg = __builtin_sqrtf(bnd ? __uint_as_float(bnd_n2) : __uint_as_float(sc.n2s) * kN2Guess) * 2.f *
                                     __builtin_sqrtf(sc.esq[kERowAnchor]) * kBetaSlack +
                                 kBetaFloor;
                const float a = __uint_as_float(sc.fbound[tid]);
                const float eg = 5.f * kUlp * (a + bg);
                const float wf = float_down(key_lower(sc.fkey[tid]) - 2.0 * ((double)bg + eg));
                sc.winf[tid] = wf;
                // a bucket reaches the window iff its upper end does: for non-NaN
                // floats a >= b iff orderable(a) >= orderable(b), once a zero
                // window takes the smaller image (-0), so both zeros pass
                sc.wkey[tid] = wf != wf ? 0xffffffffu : orderable(wf == 0.f ? -0.f : wf);
            }
            __syncthreads();
            // the lists of the (workgroup, step) pairs whose best key reaches
            // the window: entries inside it become candidates, and the
            // cutoffs bound what the lists may have left out (a workgroup
            // whose best key is outside the window has its cutoff outside
            // too, below any threshold the walk accepts)
            {
                const uint32_t wq = sk < gamma ? sc.wkey[sk] : 0xffffffffu;
                bool flag[kSumLoads];
                uint64_t lw[kSumLoads][4];
#pragma unroll
                for (int q = 0; q < kSumLoads; ++q) {
                    flag[q] = suse[q] && ready && (((uint32_t)(sw[q] >> 32) | kLidMask) >= wq);
                    const uint64_t* src =
                        regions + (flag[q] ? (int64_t)sgg[q] * kRegionWords + kListBase + kScreenStep * sk : 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        lw[q][j] = flag[q] ? __hip_atomic_load(src + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
                }
                // (the summary is written with the lists, not after them: poll
                // the few words not yet seen)
                for (int spin = 0; spin < spin_limit; ++spin) {
                    bool all = true;
#pragma unroll
                    for (int q = 0; q < kSumLoads; ++q)
#pragma unroll
                        for (int j = 0; j < 4; ++j) all = all && lw[q][j] != 0;
                    if (__all(all)) break;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int q = 0; q < kSumLoads; ++q) {
                        const uint64_t* src =
                            regions + (flag[q] ? (int64_t)sgg[q] * kRegionWords + kListBase + kScreenStep * sk : 0);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (lw[q][j] == 0) lw[q][j] = __hip_atomic_load(src + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                const uint32_t v32 = (uint32_t)V;  // V < 2^31
#pragma unroll
                for (int q = 0; q < kSumLoads; ++q) {
                    if (!flag[q]) continue;
                    bool seen = true;
#pragma unroll
                    for (int j = 0; j < 4; ++j) seen = seen && lw[q][j] != 0;
                    if (!seen) {
                        sc.abort = 1;
                        continue;
                    }
                    atomicMax(&sc.fcut[sk], (uint32_t)lw[q][3]);
#pragma unroll
                    for (int j = 0; j < kScreenEntries; ++j) {
                        const uint64_t w = lw[q][j];
                        const uint32_t id1 = (uint32_t)w;  // row id + 1, or the empty marker
                        const uint32_t qk = (uint32_t)(w >> 32);
                        if (id1 - 1u < v32 && qk != 0 && (qk | kLidMask) >= wq) {
                            const int idx = atomicAdd(&sc.ncand, 1);
                            if (idx < kCandMax) sc.cv[idx] = id1 - 1, sc.cstep[idx] = sk;
                            else sc.overflow[sk] = 1;
                        }
                    }
                }
            }
            __syncthreads();
            const bool abort = sc.abort != 0;
            const int nc = sc.ncand < kCandMax ? sc.ncand : kCandMax;
            // the real norm, posted by every row workgroup after its W2 stream:
            // a first look now, used after the table below
            const int np = tid - kChainThreads / 2;  // norm poller index
            const bool poller = !abort && np >= 0 && np + 1 < nwg;
            const uint64_t* npw = regions + (int64_t)(poller ? np + 1 : 1) * kRegionWords + kNormWord;
            uint64_t nword = poller ? __hip_atomic_load(npw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;

            // stage the candidates' rows (one wave per candidate) and forced tokens' rows
            if (!abort) {
                uint2 ra[kCandPerWave], rb[kCandPerWave];
                float cu[kCandPerWave], cg[kCandPerWave];
                // every slot's LDS words first (the slots are in range; unused
                // ones are discarded below), then every global load unconditionally
                uint32_t cvl[kCandPerWave];
                int csl[kCandPerWave];
#pragma unroll
                for (int q = 0; q < kCandPerWave; ++q) cvl[q] = sc.cv[wave + kChainWaves * q], csl[q] = sc.cstep[wave + kChainWaves * q];
                const float* gbase = G ? G : conf;  // without G: some readable word, discarded
#pragma unroll
                for (int q = 0; q < kCandPerWave; ++q) {
                    const int j = wave + kChainWaves * q;
                    const bool use = j < nc;
                    const int64_t v = use ? cvl[q] : 0;
                    const int64_t o = use ? (int64_t)csl[q] * V + v : 0;
                    ra[q] = reinterpret_cast<const uint2*>(W2 + v * kChainRank)[lane];
                    rb[q] = reinterpret_cast<const uint2*>(W1 + v * kChainRank)[lane];
                    cu[q] = load_elem(U, o);
                    const float gv = gbase[G ? o : 0];
                    cg[q] = G ? gv : 0.f;
                }
                const int kf = wave < gamma ? wave : 0;
                const int32_t f = sc.fv[kf];
                const bool fuse = wave < gamma && f >= 0 && f < V;
                const uint2 fr = reinterpret_cast<const uint2*>(W1 + (int64_t)(fuse ? f : 0) * kChainRank)[lane];
#pragma unroll
                for (int q = 0; q < kCandPerWave; ++q) {
                    const int j = wave + kChainWaves * q;
                    if (j < nc) {
                        sc.cw2[j][2 * lane] = ra[q].x, sc.cw2[j][2 * lane + 1] = ra[q].y;
                        sc.cw1[j][2 * lane] = rb[q].x, sc.cw1[j][2 * lane + 1] = rb[q].y;
                        if (lane == 0) sc.cu[j] = cu[q], sc.cg[j] = cg[q], sc.ct[j] = G ? cu[q] + cg[q] : cu[q];
                    }
                }
                if (fuse) sc.fw1[kf][2 * lane] = fr.x, sc.fw1[kf][2 * lane + 1] = fr.y;
                if (wave == 0) {
                    const int cs = lane < nc ? sc.cstep[lane] : -1;
#pragma unroll
                    for (int k = 0; k < kScreenMaxGamma; ++k) {
                        const uint32_t m = (uint32_t)__ballot(cs == k);
                        if (lane == 0) sc.stepmask[k] = m;
                    }
                }
            }
            __syncthreads();

            // every quantity the chain can need, in parallel: |e|^2 and
            // w_e . e of each e row, and W2[j] . e for each candidate j and
            // each e row that can precede its step
            // Eight lanes per dot product (the group `grp` of lane `sub`, 16
            // bf16 pairs each, then a 3-level DPP sum), so a wave forms eight
            // at once.
            if (!abort) {
                const auto erow = [&](int r) -> const uint32_t* {
                    return r < kCandMax ? sc.cw1[r] : r == kERowAnchor ? sc.e0 : sc.fw1[r - kERowForced];
                };
                const auto dot16 = [&](const uint32_t* x, const uint32_t* y) {
                    float a = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 xv = reinterpret_cast<const uint4*>(x + sub * 16)[q];
                        const uint4 yv = reinterpret_cast<const uint4*>(y + sub * 16)[q];
                        a = dot2(xv.x, yv.x, a), a = dot2(xv.y, yv.y, a), a = dot2(xv.z, yv.z, a), a = dot2(xv.w, yv.w, a);
                    }
                    return sum8(a);
                };
                for (int r = grp; r < kERows; r += kChainGroups) {  // group-uniform
                    const bool use = r < nc || r == kERowAnchor ||
                                     (r >= kERowForced && r - kERowForced < gamma && sc.fv[r - kERowForced] >= 0 &&
                                      sc.fv[r - kERowForced] < V);
                    if (!use) continue;
                    const uint32_t* er = erow(r);
                    const float es = dot16(er, er);
                    const float zc = dot16(we_lds, er);
                    if (sub == 0) sc.esq[r] = es, sc.zcm[r] = zc;
                }
                // candidate j of wave j % 8; its group g takes predecessors
                // g, g + 8, ... (in bit order)
                const int g8 = lane >> 3;
                for (int j = wave; j < nc; j += kChainWaves) {
                    const int k = sc.cstep[j];
                    uint64_t preds;  // e rows that can be e at step k
                    if (k == 0) preds = 1ull << kERowAnchor;
                    else if (sc.fv[k - 1] >= 0) preds = 1ull << (kERowForced + k - 1);
                    else preds = sc.stepmask[k - 1];
                    for (int t = 0; t < g8; ++t) preds &= preds - 1;
                    while (preds) {  // group-uniform
                        const int r = __builtin_ctzll(preds);
                        const float b = dot16(sc.cw2[j], erow(r));
                        if (sub == 0) sc.bias[j][r] = b;
                        for (int t = 0; t < 8; ++t) preds &= preds - 1;
                    }
                }
            }
            // The walk.  Every step's winner depends on the step before only
            // through the e row that precedes it, so first a table: for each
            // step k and each e row r that can precede it, the bound check and
            // the best candidate (one thread per pair).  The walk itself is then
            // a chain of lookups in wave 0.  It first runs with the guessed
            // largest row norm while waves 4-7 collect the real one; a guess at
            // least as large makes the candidate sets supersets of the exact
            // ones, inside the windows, so the result stands when the real norm
            // is no larger.  Otherwise table and walk run again.
            __syncthreads();  // the bias table is complete
            // a second look at the norms (the streams end about now), read after the walk
            if (poller && nword == 0) nword = __hip_atomic_load(npw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // one thread per (step, e row) pair; every LDS read of a pair is
            // issued before the first is used, and the candidates of a step
            // come four at a time (a repeated last index is harmless: its
            // key is never strictly larger)
            static_assert(kScreenMaxGamma * kERows <= kChainThreads, "one pair per thread");
            const auto build = [&](uint32_t n2b) {
                if (tid >= gamma * kERows) return;
                const int k = tid / kERows, r = tid - k * kERows;
                const int32_t fprev = sc.fv[k > 0 ? k - 1 : 0];
                const int32_t fk = sc.fv[k];
                const int csr = sc.cstep[r < kCandMax ? r : 0];
                const uint32_t m = sc.stepmask[k];
                const float es = sc.esq[r];
                const uint32_t ab = sc.fbound[k];
                const uint32_t cut = sc.fcut[k];
                const int ovf = sc.overflow[k];
                const float wf = sc.winf[k];
                // r can be the e row of step k
                const bool pv = k == 0 ? r == kERowAnchor
                                       : fprev >= 0 ? r == kERowForced + k - 1 : r < nc && csr == k - 1;
                const auto four = [](uint32_t& bits, int (&js)[4]) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        js[u] = bits ? __builtin_ctz(bits) : js[0];
                        bits &= bits - 1;
                    }
                };
                int bj = -1;
                int32_t bt = -1;
                if (pv && !abort) {
                    float tmax = -__builtin_inff();
                    for (uint32_t bits = m; bits;) {
                        int js[4];
                        four(bits, js);
                        float a[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) a[u] = sc.ct[js[u]];
                        tmax = fmaxf(tmax, fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])));
                    }
                    const float n2 = __builtin_sqrtf(__uint_as_float(n2b));
                    const float beta = n2 * __builtin_sqrtf(es) * kBetaSlack + kBetaFloor;
                    const float eps = 5.f * kUlp * (__uint_as_float(ab) + beta);
                    const double thr = (double)tmax - 2.0 * ((double)beta + eps);
                    const bool ok = ovf == 0 && finite_bits(ab) && finite_bits(n2b) && finite_bits(bound_bits(es)) &&
                                    tmax > -__builtin_inff() && thr >= (double)wf && key_upper(cut) < thr;
                    if (ok) {
                        uint64_t best = 0;
                        for (uint32_t bits = m; bits;) {
                            int js[4];
                            four(bits, js);
                            float c4[4], u4[4], b4[4], g4[4];
                            uint32_t v4[4];
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                c4[u] = sc.ct[js[u]], u4[u] = sc.cu[js[u]], b4[u] = sc.bias[js[u]][r];
                                g4[u] = G ? sc.cg[js[u]] : 0.f, v4[u] = sc.cv[js[u]];
                            }
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const float lg = u4[u] + b4[u];
                                const uint64_t key = (double)c4[u] >= thr ? argmax_key(G ? lg + g4[u] : lg, v4[u]) : 0;
                                if (key > best) best = key, bj = js[u];
                            }
                        }
                        // the best listed row is always a candidate, so best != 0
                        bt = best != 0 ? key_token(best) : -1;
                        if (best == 0) bj = -1;
                    }
                }
                const int64_t xk = fk >= 0 ? fk : bt;
                const int nx = bj < 0 ? -1 : !(xk >= 0 && xk < V) ? -2 : fk >= 0 ? kERowForced + k : bj;
                sc.tjt[k][r] = make_int2(nx, bt);
            };
            struct Walk {
                int k, pst;
                int32_t tk;
                int64_t x;
                bool valid, fail;
            };
            // the walk in wave 0: lane r holds column r of the table, and the
            // chain follows it with lane reads (the e row is wave-uniform);
            // lane k keeps step k's e row and token
            const auto walk = [&]() {
                Walk w{0, 0, -1, xa, true, sc.abort != 0};
                int2 col[kScreenMaxGamma];
#pragma unroll
                for (int k = 0; k < kScreenMaxGamma; ++k) col[k] = sc.tjt[k][lane < kERows ? lane : 0];
                const int32_t fl = sc.fv[lane < kScreenMaxGamma ? lane : 0];
                bool run = !w.fail;
                int cur = kERowAnchor;  // e row of the current step
                int last = -1;          // last step with a sampled token
#pragma unroll
                for (int k = 0; k < kScreenMaxGamma; ++k) {
                    if (run && k < gamma) {  // wave-uniform
                        const int nx = __builtin_amdgcn_readlane(col[k].x, cur);
                        if (nx == -1) {
                            w.fail = true;
                            run = false;
                        } else {
                            const int32_t tok = __builtin_amdgcn_readlane(col[k].y, cur);
                            if (lane == k) w.pst = cur, w.tk = tok;
                            last = k;
                            run = nx >= 0;
                            w.valid = run;
                            w.k = run ? k + 1 : gamma;  // past an invalid token the steps are idle
                            cur = nx;
                        }
                    }
                }
                if (last >= 0) {
                    const int32_t f = __builtin_amdgcn_readlane(fl, last);
                    w.x = f >= 0 ? f : __builtin_amdgcn_readlane(w.tk, last);
                }
                return w;
            };
            // with a bound whose sampled rows' norm differs from this W2's,
            // the weights changed after it was computed: nothing is proved
            // from it, and the whole block takes the per-step exchange
            const bool stale = bnd && sc.n2s != bnd_n2s;  // workgroup-uniform
            if (tid == 0 && bnd) mark_path(header, stale ? kPathB1BoundStale : kPathB1Bound);
            const float guess = bnd ? __uint_as_float(bnd_n2) : __uint_as_float(sc.n2s) * kN2Guess;
            if (!stale) build(bound_bits(guess));
            __syncthreads();
            Walk wk{0, 0, -1, xa, true, true};
            if (wave == 0 && !stale) wk = walk();
            uint32_t nmine = 0;
            if (poller) {
                uint64_t w = nword;
                for (int spin = 0; spin < spin_limit && w == 0; ++spin) {
                    __builtin_amdgcn_s_sleep(1);
                    w = __hip_atomic_load(npw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (w == 0) sc.abort = 1;
                nmine = (uint32_t)w;
            }
            if (wave >= kChainWaves / 2) {  // the pollers' waves: one LDS atomic each
                const uint32_t wm = wave_max_u32(nmine);
                if (lane == 0 && wm != 0) atomicMax(&sc.n2, wm);
            }
            __syncthreads();
            const uint32_t n2b = sc.n2;
            if (!stale && (sc.abort || !(__uint_as_float(n2b) <= guess))) {  // workgroup-uniform
                if (tid == 0 && !sc.abort) mark_path(header, kPathB1Rebuild);
                build(n2b);
                __syncthreads();
                if (wave == 0) wk = walk();
            }
            if (wave == 0) {
                const int k = wk.k;
                const bool fail = wk.fail;
                const int pst = wk.pst;
                const int32_t tk = wk.tk;
                x = wk.x;
                valid = wk.valid;
                // the decision first (it needs no confidence), so the row
                // workgroups are released while this wave writes the outputs
                const uint64_t d = (fail && !sc.abort)
                                       ? (kDecideResume | ((uint64_t)k << 32) | (uint64_t)(uint32_t)x)
                                       : kDecideDone;
                if (lane == 0) sc.decision = d;
                // (only the copies some row workgroup reads: each is cleared by its last reader)
                if (lane < kCopies && (lane == 0 ? kCopies : lane) < nwg)
                    __hip_atomic_store(aux + lane * kSlotWords, d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                // confidences of the settled steps in parallel, then the running product
                const int settled = k;
                float c = 0.f;
                if (lane < settled && tk >= 0)
                    c = 1.f / (1.f + expf(-(sc.pk[lane] + sc.zcm[pst] + b_conf)));
                if (lane < settled) tokens[lane] = tk;
                float surv = 1.f;
                bool alive = true;
#pragma unroll
                for (int q = 0; q < kScreenMaxGamma; ++q) {
                    if (q < settled) {  // wave-uniform
                        const float cq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), q));
                        alive = alive && __builtin_amdgcn_readlane(tk, q) >= 0;
                        surv = surv * cq;
                        if (lane == q) {
                            conf[q] = alive ? cq : __builtin_nanf("");
                            survival[q] = alive ? surv : __builtin_nanf("");
                        }
                    }
                }
                if (lane == 0) A = surv;
                if (sc.abort) {  // some workgroup never arrived: report, release the others
                    if (lane == 0) mark_gave_up(header);
                    for (int j = lane; j < gamma; j += 64)
                        tokens[j] = -1, conf[j] = __builtin_nanf(""), survival[j] = __builtin_nanf("");
                }
            }
            __syncthreads();
            const uint64_t d = sc.decision;
            if (d & kDecideDone) {
                // each row workgroup clears its own region once it has read
                // the decision, and the last reader of each decision copy
                // clears that copy: nothing is left to wait for here
                done = true;
            } else {
                k0 = (int)((d >> 32) & 0xffff);
                x = (int32_t)(uint32_t)d;
                valid = true;
            }
        }
    } else if (scr) {
        if (tid < kScreenMaxGamma) sc.a1[tid] = 0;
        if (tid == 0) sc.sync = 0;
        __syncthreads();
        if (wave < kScreenWaves) {
            // Screening waves: nothing of W2 is in flight here, so every wait
            // for a small load is exact.  Lane i screens rows i, i + 256, ...
            int64_t sv[kScreenRows];
            bool sok[kScreenRows];
            uint16_t ur[kScreenMaxGamma][kScreenRows];
            float gs[kScreenMaxGamma][kScreenRows];
#pragma unroll
            for (int m = 0; m < kScreenRows; ++m) {
                const int lr = tid + kScreenLanes * m;
                sv[m] = row0 + lr;
                sok[m] = lr < rows_per_wg && sv[m] < V;
            }
#pragma unroll
            for (int k = 0; k < kScreenMaxGamma; ++k)
#pragma unroll
                for (int m = 0; m < kScreenRows; ++m) {
                    const int64_t o = (k < gamma && sok[m]) ? (int64_t)k * V + sv[m] : 0;
                    ur[k][m] = U[o].bits;
                    gs[k][m] = G ? G[o] : 0.f;
                }
            // each wave's four best ranking keys and |U|+|G| bound per step
#pragma unroll
            for (int k = 0; k < kScreenMaxGamma; ++k) {
                if (k >= gamma) break;
                uint32_t q[kScreenRows];  // this lane's keys, best first
                uint32_t am = 0;
#pragma unroll
                for (int m = 0; m < kScreenRows; ++m) {
                    const float u = __uint_as_float((uint32_t)ur[k][m] << 16);
                    am = sok[m] ? max(am, bound_bits(__builtin_fabsf(u) + __builtin_fabsf(gs[k][m]))) : am;
                    q[m] = sok[m] ? ranking_key(G ? u + gs[k][m] : u, (uint32_t)(sv[m] - row0)) : 0u;
                }
#pragma unroll
                for (int i = 0; i < kScreenRows; ++i)  // sort descending
#pragma unroll
                    for (int j = kScreenRows - 1; j > i; --j) {
                        const uint32_t hi = max(q[j - 1], q[j]), lo = min(q[j - 1], q[j]);
                        q[j - 1] = hi, q[j] = lo;
                    }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t mr = wave_max_u32(q[0]);
                    if (q[0] == mr) {
#pragma unroll
                        for (int m = 0; m + 1 < kScreenRows; ++m) q[m] = q[m + 1];
                        q[kScreenRows - 1] = 0;
                    }
                    if (lane == 0) sc.wtop[k][wave][r] = mr;
                }
                am = wave_max_u32(am);
                if (lane == 0) atomicMax(&sc.a1[k], am);
            }
            screen_sync(sc, lane, kScreenWaves);
            // wave w merges steps w, w + 4 and publishes their list words
            // and their summary word each
#pragma unroll
            for (int k = wave; k < kScreenMaxGamma; k += kScreenWaves) {
                if (k >= gamma) break;
                uint32_t c = lane < 4 * kScreenWaves ? sc.wtop[k][lane >> 2][lane & 3] : 0u;
                uint32_t t4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    t4[r] = wave_max_u32(c);
                    if (c == t4[r]) c = 0;
                }
                const uint32_t te = lane == 0 ? t4[0] : lane == 1 ? t4[1] : t4[2];
                uint64_t word;
                if (lane < kScreenEntries)
                    word = te ? (((uint64_t)te << 32) | (uint64_t)(row0 + (te & kLidMask) + 1)) : kEmptyEntry;
                else if (lane == 3)
                    word = kTag | t4[3];
                else
                    word = ((uint64_t)t4[0] << 32) | (sc.a1[k] | 1u);
                if (lane < kScreenStep)
                    __hip_atomic_store(myregion + kListBase + kScreenStep * k + lane, word, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                else if (lane == kScreenStep)
                    __hip_atomic_store(myregion + k, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            screen_sync(sc, lane, 2 * kScreenWaves);
        } else {
            // Norm waves: the W2 slice streams through a window of slots for
            // the largest squared row norm, at the throttled rate described
            // above (the remaining waves idle here).  Rows past the slice
            // load row 0 and are masked out (a zero fill would wait for the
            // load it overwrites).
            const int ng = (tid - kScreenLanes) >> 3;
            constexpr int NS = (NSLOT * kChainGroups + kNormGroups - 1) / kNormGroups;
            uint32_t nb = 0;
            if (!bnd && tid < kScreenLanes + kNormLanes) {
                uint32_t buf[kStreamSlots][16];
#pragma unroll
                for (int i = 0; i < kStreamSlots; ++i) {
                    const int lr = i * kNormGroups + ng;
                    const bool in = i < NS && lr < rows_per_wg && row0 + lr < V;
                    load64B(W2 + (in ? row0 + lr : 0) * kChainRank + sub * 32, buf[i]);
                }
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    float a = 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) a = dot2(buf[i % kStreamSlots][q], buf[i % kStreamSlots][q], a);
                    a = sum8(a);
                    const int lr = i * kNormGroups + ng;
                    if (lr < rows_per_wg && row0 + lr < V) nb = max(nb, bound_bits(a));
                    if (i + kStreamSlots < NS) {
                        const int lr2 = (i + kStreamSlots) * kNormGroups + ng;
                        const bool in = lr2 < rows_per_wg && row0 + lr2 < V;
                        load64B(W2 + (in ? row0 + lr2 : 0) * kChainRank + sub * 32, buf[i % kStreamSlots]);
                    }
                }
            }
            nb = wave_max_u32(nb);
            if (lane == 0) sc.wn[wave] = nb;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t m = 0;
#pragma unroll
            for (int w = kScreenWaves; w < kChainWaves; ++w) m = max(m, sc.wn[w]);
            if (bnd) m = bnd_n2;  // (no stream ran)
            __hip_atomic_store(myregion + kNormWord, kTag | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // wait for the coordinator's decision
            uint64_t d = 0;
            for (int spin = 0; spin < spin_limit && d == 0; ++spin) {
                d = __hip_atomic_load(dcopy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (d == 0) __builtin_amdgcn_s_sleep(2);
            }
            if (d == 0) mark_gave_up(header);  // the coordinator was lost
            if (d & kDecideDone) {
                // count out on this copy (word 1 beside the decision); its
                // last reader clears both words.  The decision was read above,
                // before the count.  (Readers of copy c: the workgroups
                // g >= 1 with g % kCopies == c.)
                const int c = g % kCopies;
                const int g0 = c == 0 ? kCopies : c;
                const uint64_t readers = (uint64_t)((nwg - 1 - g0) / kCopies + 1);
                const uint64_t prev = __hip_atomic_fetch_add(dcopy + 1, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (prev + 1 == readers) {
                    __hip_atomic_store(dcopy + 1, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(dcopy, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            sc.decision = d;
        }
        __syncthreads();
        const uint64_t d = sc.decision;
        if (tid < kRegionUsed)  // read by the coordinator before it decided
            __hip_atomic_store(myregion + tid, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0 || (d & kDecideDone)) {
            done = true;
        } else {
            k0 = (int)((d >> 32) & 0xffff);
            x = (int32_t)(uint32_t)d;
            valid = true;
        }
    }

    if (done) return;  // settled by the screen: no slots were written, the regions are clear

    // the per-step exchange keeps this workgroup's W2 rows in registers
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
        const int lr = i * kChainGroups + grp;
        const int64_t v = row0 + lr;
        if (lr < rows_per_wg && v < V) {
            load64B(W2 + v * kChainRank + sub * 32, w2[i]);
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) w2[i][q] = 0u;
        }
    }

    {
        // the grid-wide per-step exchange, from step k0 on
        if (wg0 && tid == 0) mark_path(header, kPathB1Exchange);
        uint32_t e[16];
        if (valid) load64B(W1 + x * kChainRank + sub * 32, e);
        float u_next[NMINE], g_next[NMINE];
#pragma unroll
        for (int m = 0; m < NMINE; ++m) {
            const int64_t o = my_ok[m] ? (int64_t)k0 * V + my_v[m] : 0;
            u_next[m] = load_elem(U, o);
            g_next[m] = G ? G[o] : 0.f;
        }
        __syncthreads();

        for (int k = k0; k < gamma; ++k) {
            if (!valid) {  // identical in every workgroup: no exchange needed
                if (wg0 && tid == 0) tokens[k] = -1, conf[k] = __builtin_nanf(""), survival[k] = __builtin_nanf("");
                continue;
            }
            // this workgroup's share of the confidence logit: a slice of w_h . h_k
            // (loaded here, summed after the dot products), plus (workgroup 0) the
            // Markov part w_e . e
            float p = 0.f;
            for (int64_t i = h_lo + tid; i < h_hi; i += kChainThreads)
                p += load_elem(w_conf, i) * load_elem(h, (int64_t)k * H + i);
            float acc[NSLOT];
#pragma unroll
            for (int i = 0; i < NSLOT; ++i) {
                float a = 0.f;
#pragma unroll
                for (int q = 0; q < 16; ++q) a = dot2(w2[i][q], e[q], a);
                acc[i] = sum8(a);
            }
            uint64_t key = 0;
#pragma unroll
            for (int m = 0; m < NMINE; ++m) {
                float bias = 0.f;
#pragma unroll
                for (int i = 0; i < NSLOT; ++i) bias = (sub + 8 * m == i) ? acc[i] : bias;
                if (my_ok[m]) {
                    const float lg = u_next[m] + bias;
                    const float sc2 = G ? lg + g_next[m] : lg;
                    if (bias_out) bias_out[(int64_t)k * V + my_v[m]] = bias;
                    if (logits_out) logits_out[(int64_t)k * V + my_v[m]] = lg;
                    key = umax64(key, argmax_key(sc2, (uint32_t)my_v[m]));
                }
                // next step's inputs do not depend on this step's token; loaded
                // unconditionally from a clamped index so nothing waits for them here
                const int64_t on = (my_ok[m] && k + 1 < gamma) ? (int64_t)(k + 1) * V + my_v[m] : 0;
                u_next[m] = load_elem(U, on);
                if (G) g_next[m] = G[on];
            }
            if (wg0 && tid < 8)
#pragma unroll
                for (int q = 0; q < 16; ++q) p = dot2(we_lds[tid * 16 + q], e[q], p);
            p = wave_sum_f32(p);
            key = wave_max_u64(key);
            if (lane == 0) red[wave] = key, fred[wave] = p;
            __syncthreads();
            if (tid == 0) {
                uint64_t m = 1;  // a workgroup without rows still publishes a non-zero key
                float ps = 0.f;
#pragma unroll
                for (int w = 0; w < kChainWaves; ++w) m = umax64(m, red[w]), ps += fred[w];
                uint64_t* slot = slots + ((int64_t)k * nwg + g) * kSlotWords;
                __hip_atomic_store(slot, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot + 1, (1ull << 32) | __float_as_uint(ps), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }

            if (wave == 0) {
                uint64_t best = 0;
                float zsum = 0.f;
                for (int spin = 0; spin < spin_limit; ++spin) {
                    uint64_t sk[kChainPoll], sp[kChainPoll];
#pragma unroll
                    for (int i = 0; i < kChainPoll; ++i) {  // clamped, unconditional: all in flight at once
                        const int j = lane + 64 * i;
                        const uint64_t* slot = slots + ((int64_t)k * nwg + (j < nwg ? j : 0)) * kSlotWords;
                        const uint64_t a = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const uint64_t b = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        sk[i] = j < nwg ? a : 1ull;
                        sp[i] = j < nwg ? b : (1ull << 32);
                    }
                    bool all = true;
                    uint64_t m = 0;
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < kChainPoll; ++i) {
                        all = all && sk[i] != 0 && sp[i] != 0;
                        m = umax64(m, sk[i]);
                        ps += __uint_as_float((uint32_t)sp[i]);
                    }
                    if (__all(all)) {
                        best = wave_max_u64(m);
                        zsum = wave_sum_f32(ps);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (lane == 0) {
                    winner = best;
                    zpart = zsum;
                    if (best == 0) mark_gave_up(header);  // timed out: reported as token -1
                }
            }
            __syncthreads();
            const uint64_t wk = winner;
            if (wg0 && tid == 0) {
                const float c = 1.f / (1.f + expf(-(zpart + b_conf)));
                A = A * c;
                conf[k] = c;
                survival[k] = A;
            }
            const int32_t tok = key_token(wk);
            const int32_t f = (force && wk != 0) ? force[k] : -1;
            x = f >= 0 ? f : tok;
            valid = wk != 0 && x >= 0 && x < V;
            if (valid && k + 1 < gamma) load64B(W1 + x * kChainRank + sub * 32, e);
            if (wg0 && tid == 0) {
                tokens[k] = tok;
                if (wk == 0) conf[k] = __builtin_nanf(""), survival[k] = __builtin_nanf("");
            }
        }
    }

    // leave: the last workgroup out clears the slots and the decision word for the next call
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&header[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == (uint32_t)(nwg - 1);
    }
    __syncthreads();
    if (last_flag) {
        for (int64_t i = tid; i < (int64_t)gamma * nwg; i += kChainThreads) {
            __hip_atomic_store(&slots[i * kSlotWords], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&slots[i * kSlotWords + 1], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) {
            for (int c = 0; c < kCopies; ++c)
                __hip_atomic_store(aux + c * kSlotWords, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&header[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// The weights-only bound of the B = 1 screen (dspark_w2_bound): the largest
// squared W2 row norm, with the same per-row arithmetic as the norm stream
// (eight lanes per row, 32 rank elements each, dot2 then sum8), so the
// screen proves exactly what the stream would have let it prove; and a
// fingerprint (the coordinator's sample of 64 rows, computed exactly as the
// coordinator does, plus V, the rank and the address of W2).
//   out[0] largest bound_bits of a row's squared norm   out[1] that of the sample
//   out[2], out[3] V   out[4] rank   out[5], out[6] address of W2   out[7] kW2BoundTag
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kChainThreads) void w2_bound_init(int64_t V, const bf16_t* __restrict__ W2,
                                                                uint32_t* __restrict__ out) {
    __shared__ uint32_t wn[kChainWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = tid >> 3, sub = tid & 7;
    uint32_t smp[16];
    load64B(W2 + (int64_t)grp * (V / kSampleRows) * kChainRank + sub * 32, smp);
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) a = dot2(smp[q], smp[q], a);
    const uint32_t m = wave_max_u32(bound_bits(sum8(a)));
    if (lane == 0) wn[wave] = m;
    __syncthreads();
    if (tid == 0) {
        uint32_t n2s = 0;
#pragma unroll
        for (int w = 0; w < kChainWaves; ++w) n2s = max(n2s, wn[w]);
        const uint64_t addr = (uint64_t)(uintptr_t)W2;
        out[0] = 0u;
        out[1] = n2s;
        out[2] = (uint32_t)V;
        out[3] = (uint32_t)((uint64_t)V >> 32);
        out[4] = (uint32_t)kChainRank;
        out[5] = (uint32_t)addr;
        out[6] = (uint32_t)(addr >> 32);
        out[7] = 0u;
    }
}

__global__ __launch_bounds__(kChainThreads) void w2_bound_max(int64_t V, const bf16_t* __restrict__ W2,
                                                               uint32_t* __restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 3, sub = tid & 7;
    uint32_t nb = 0;
    // 4 x 64 rows per workgroup and round, all four loads of a lane in
    // flight together; a row's eight lanes are consecutive
    constexpr int kU = 4;
    for (int64_t v0 = (int64_t)blockIdx.x * kSampleRows * kU + grp; v0 < V;
         v0 += (int64_t)gridDim.x * kSampleRows * kU) {
        uint32_t b[kU][16];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t v = v0 + (int64_t)u * kSampleRows;
            load64B(W2 + (v < V ? v : 0) * kChainRank + sub * 32, b[u]);  // past V: row 0, unused
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) a = dot2(b[u][q], b[u][q], a);
            a = sum8(a);
            if (v0 + (int64_t)u * kSampleRows < V) nb = max(nb, bound_bits(a));
        }
    }
    nb = wave_max_u32(nb);
    if (lane == 0 && nb != 0) __hip_atomic_fetch_max(out, nb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void w2_bound_tag(uint32_t* __restrict__ out) {
    if (threadIdx.x == 0) out[7] = kW2BoundTag;
}

const void* chain_fn(int nslot) {
    switch (nslot) {
        case 1: return reinterpret_cast<const void*>(&sample_chain_b1<1>);
        case 2: return reinterpret_cast<const void*>(&sample_chain_b1<2>);
        case 3: return reinterpret_cast<const void*>(&sample_chain_b1<3>);
        case 4: return reinterpret_cast<const void*>(&sample_chain_b1<4>);
        case 5: return reinterpret_cast<const void*>(&sample_chain_b1<5>);
        case 6: return reinterpret_cast<const void*>(&sample_chain_b1<6>);
        case 7: return reinterpret_cast<const void*>(&sample_chain_b1<7>);
        case 8: return reinterpret_cast<const void*>(&sample_chain_b1<8>);
        case 9: return reinterpret_cast<const void*>(&sample_chain_b1<9>);
        default: return reinterpret_cast<const void*>(&sample_chain_b1<10>);
    }
}

struct ChainPlan {
    int nwg = 0, rows_per_wg = 0, nslot = 0;
};

// Number of compute units of the current device (queried once per device).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// Workgroup 0 coordinates; workgroups 1.. hold the vocabulary rows.
ChainPlan chain_plan(int64_t V, int64_t H) {
    ChainPlan p;
    const int cus = device_cus();
    if (cus < 2) return p;
    int64_t nrow = (V + kChainGroups - 1) / kChainGroups;  // at least one full slot of rows per workgroup
    if (nrow > cus - 1) nrow = cus - 1;
    if (nrow > kChainMaxWGs - 1) nrow = kChainMaxWGs - 1;
    const int64_t rows = (V + nrow - 1) / nrow;
    const int64_t nslot = (rows + kChainGroups - 1) / kChainGroups;
    if (nslot > kChainMaxSlots) return p;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_fn((int)nslot), kChainThreads, 0) != hipSuccess ||
        per_cu < 1)
        return p;
    p.nwg = (int)nrow + 1;
    p.rows_per_wg = (int)rows;
    p.nslot = (int)nslot;
    return p;
}

size_t chain_workspace(int64_t gamma) {
    return kChainHeader + (size_t)8 * kSlotWords * gamma * kChainMaxWGs + (size_t)8 * kRegionWords * kChainMaxWGs +
           (size_t)8 * kAuxWords;
}

hipError_t launch_chain(const ChainPlan& p, int64_t gamma, int64_t V, int64_t H, const void* U, const void* h,
                        const void* W1, const void* W2, const void* w_conf, float b_conf, const int32_t* x0,
                        const float* G, const int32_t* force, int32_t* tokens, float* conf, float* survival,
                        float* lo, float* bo, void* ws, hipStream_t stream, const uint32_t* nbound) {
    int g = (int)gamma;
    int64_t Vv = V, Hh = H;
    int rows = p.rows_per_wg;
    // the screen needs every step's U and G in registers and no full logit rows requested
    int screen = (gamma <= kScreenMaxGamma && lo == nullptr && bo == nullptr) ? 1 : 0;
    const bf16_t* Ut = static_cast<const bf16_t*>(U);
    const bf16_t* ht = static_cast<const bf16_t*>(h);
    const bf16_t* W1t = static_cast<const bf16_t*>(W1);
    const bf16_t* W2t = static_cast<const bf16_t*>(W2);
    const bf16_t* wt = static_cast<const bf16_t*>(w_conf);
    uint32_t* header = static_cast<uint32_t*>(ws);
    uint64_t* slots = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kChainHeader);
    uint64_t* regions = slots + (size_t)kSlotWords * gamma * kChainMaxWGs;
    uint64_t* aux = regions + (size_t)kRegionWords * kChainMaxWGs;
    int lim = wait_limit(kChainSpinLimit);
    void* args[] = {&g,     &Vv,    &Hh,       &rows, &screen, &Ut,    &ht,      &W1t, &W2t,    &wt,   &b_conf, &x0,
                    &G,     &force, &tokens,   &conf, &survival, &lo,  &bo,      &slots, &regions, &aux, &header, &lim,
                    &nbound};
    const void* fn = chain_fn(p.nslot);
    // A plain launch: every workgroup needs a whole CU (its register file) and
    // the grid has at most one workgroup per CU, so on an otherwise idle GPU
    // all of them are resident together.  The planner checked that one fits
    // per CU; the bounded spins turn any other outcome into an error, not a
    // hang.
    return hipLaunchKernel(fn, dim3(p.nwg), dim3(kChainThreads), args, 0, stream);
}



// ---------------------------------------------------------------------------
// Batched step kernel on the matrix cores (bf16, rank 256).
//
// The bias of a whole step is the product W2[V, 256] . E^T[256, B], E = the
// gathered W1 rows of the requests' previous tokens.  Each workgroup takes 128
// vocabulary rows and up to 64 requests; each wave multiplies its 32 rows by
// the requests with v_mfma_f32_32x32x16_bf16 (W2 rows as the A operand, E^T
// as B), straight from HBM; the B operand comes from E in LDS.
// The accumulator layout leaves each lane with 16 vocabulary rows of one
// request, so the +U (+G) epilogue and the argmax are in-lane, then one swap
// between lane halves and a 4-wave reduction in LDS.  The workgroup's U and G
// tiles (64 requests x 128 rows) are fetched with coalesced 16-byte loads
// before the products and parked in LDS (in E's space) for the epilogue; with
// rows that are not 16-byte aligned each lane reads its own elements.  The
// [B x V] bias never reaches HBM.  Keys go to one of 16 copies by workgroup,
// to spread atomics.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16 bytes as a first-class vector: staged copies global -> registers -> LDS
// stay in registers (a uint4 struct copy becomes a memcpy through scratch)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaRank = 256;
constexpr int kMfmaRows = 128;      // vocabulary rows per workgroup (32 per wave)
constexpr int kKeyCopies = 16;
constexpr int kMfmaMinBatch = 16;   // smaller batches stay on the vector path
constexpr int kERow = kMfmaRank + 8;  // LDS row stride of E in bf16 (padding against bank conflicts)

constexpr int kURow = kMfmaRows + 8;   // LDS row stride of the U tile (bf16)
constexpr int kGRow = kMfmaRows + 4;   // LDS row stride of the G tile (fp32)

// Hidden halves of the gated and RNN heads on the matrix cores (bf16):
//   out_z[bk][j] = W_z[j, off : off + H] . h[bk, :]   for bk < M = B gamma, j < r
// with z choosing (Wa, outa) or (Wb, outb); W rows have stride ld.  grid
// (r / 32, ceil(M / 32), (1 or 2) KS), 512 threads, blockIdx.z = z KS + ks: a
// workgroup owns a 32 x 32 output tile and the ks-th of KS equal ranges of
// the k-steps (of 32 each), its eight waves take interleaved runs of KU
// k-steps (the loads of a run are all in flight at once), and the eight
// partial tiles are summed in wave order (deterministic).  The products are
// v_mfma_f32_16x16x32_bf16, four per k-step (two 16-row halves of W times two
// of h): lane l holds 8 consecutive k of row l % 16, so the four lanes of a
// row read 64 contiguous bytes and a load instruction fills 16 whole cache
// lines.  Range ks goes to out_z + ks M r, as [M][r] or, with colmajor,
// [r][M] (each column contiguous); the KS partials are summed by the
// consumer.  Requires r % 32 == 0, H % 32 == 0, ld % 8 == 0, off % 8 == 0 and
// 16-byte aligned W and h.
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
constexpr int kHidWaves = 8;
#ifndef DSPARK_HID_KU
#define DSPARK_HID_KU 4
#endif
constexpr int kHidKU = DSPARK_HID_KU;  // k-steps of 32 per run: 16 loads of 16 bytes in flight per lane
template <int KU>
__global__ __launch_bounds__(64 * kHidWaves) void hidden_mfma(int64_t M, int64_t H, int64_t r, int64_t ld,
                                                              int64_t off, const bf16_t* __restrict__ h,
                                                              const bf16_t* __restrict__ Wa,
                                                              const bf16_t* __restrict__ Wb, float* __restrict__ outa,
                                                              float* __restrict__ outb, int KS, int colmajor) {
    __shared__ float part[kHidWaves][16 * 64];
    // the wave index as a scalar: the k-step guards below are then uniform branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = lane & 15, kq = lane >> 4;
    const int zm = (int)blockIdx.z / KS, ks = (int)blockIdx.z % KS;
    const bf16_t* W = zm ? Wb : Wa;
    float* out = (zm ? outb : outa) + (int64_t)ks * M * r;
    // Workgroups go round-robin over the 8 XCDs (each with its own L2); when
    // the tile count allows, XCD x takes the x-th eighth of the tiles in
    // row-major order, so it reads a few h rows and W once instead of all of h.
    const uint32_t nj = gridDim.x, T = gridDim.x * gridDim.y, L = blockIdx.x + nj * blockIdx.y;
    const uint32_t t = T % 8 == 0 ? (L % 8) * (T / 8) + L / 8 : L;
    const int64_t j0 = (int64_t)(t % nj) * 32, m0 = (int64_t)(t / nj) * 32;
    int64_t mr[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) mr[q] = m0 + 16 * q + row < M ? m0 + 16 * q + row : M - 1;  // clamped: never stored
    const uint4* ap[2];
    const uint4* bp[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        ap[q] = reinterpret_cast<const uint4*>(W + (j0 + 16 * q + row) * ld + off + kq * 8);
        bp[q] = reinterpret_cast<const uint4*>(h + mr[q] * H + kq * 8);
    }
    const int nsteps = (int)(H / 32);
    const int s_lo = (int)((int64_t)nsteps * ks / KS), steps = (int)((int64_t)nsteps * (ks + 1) / KS);
    f32x4v_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const uint4 (&a)[2], const uint4 (&b)[2]) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
                acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[x]),
                                                                   __builtin_bit_cast(bf16x8_t, b[y]), acc[x][y], 0,
                                                                   0, 0);
    };
    constexpr int kU = KU;  // k-steps in flight per wave
    int s0 = s_lo + wave * kU;
    for (; s0 + kU <= steps; s0 += kHidWaves * kU) {  // whole runs, no guards
        uint4 a[kU][2], b[kU][2];
#pragma unroll
        for (int i = 0; i < kU; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q) a[i][q] = ap[q][4 * (s0 + i)], b[i][q] = bp[q][4 * (s0 + i)];
        __builtin_amdgcn_sched_barrier(0);  // every load of the run issued before the first product
#pragma unroll
        for (int i = 0; i < kU; ++i) step(a[i], b[i]);
    }
    for (int s = s0; s < steps && s < s0 + kU; ++s) {  // the one partial run, if any
        const uint4 a[2] = {ap[0][4 * s], ap[1][4 * s]}, b[2] = {bp[0][4 * s], bp[1][4 * s]};
        step(a, b);
    }
    // register i = 4 (2 x + y) + e of lane l: W row j0 + 16 x + 4 (l / 16) + e, h row m0 + 16 y + l % 16
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[wave][(4 * (2 * x + y) + e) * 64 + lane] = acc[x][y][e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16 * 64 / (64 * kHidWaves); ++q) {
        const int el = tid + 64 * kHidWaves * q, i = el >> 6, l = el & 63;
        float v = part[0][el];
#pragma unroll
        for (int w = 1; w < kHidWaves; ++w) v += part[w][el];
        const int x = i >> 3, y = (i >> 2) & 1, e = i & 3;
        const int64_t m = m0 + 16 * y + (l & 15), j = j0 + 16 * x + 4 * (l >> 4) + e;
        if (m < M) out[colmajor ? j * M + m : m * r + j] = v;
    }
}

// split-K ranges of the hidden halves (at most kHidMaxSplits): the gated
// head's single matrix makes only r / 32 x ceil(B gamma / 32) tiles (112
// workgroups at B gamma = 448), so two ranges, each with a whole run per
// wave, bring more compute units in; the RNN head's two matrices already fill
// the chip
constexpr int kHidMaxSplits = 2;
int hidden_splits(int64_t H, int hd) { return hd == 1 && H / 32 >= 2 * kHidWaves * kHidKU ? 2 : 1; }

bool hidden_mfma_ok(int64_t H, int64_t r, int64_t ld, int64_t off, const void* h, const void* W) {
    return H > 0 && H % 32 == 0 && r % 32 == 0 && ld % 8 == 0 && off % 8 == 0 && (uintptr_t)h % 16 == 0 &&
           (uintptr_t)W % 16 == 0;
}

// bf16 bits of a finite binary32 value, rounded to nearest even
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// EG: the embedding of a gated or RNN head is a binary32 vector per request
// (eg [B][256]), not a bf16 row of W1.  It enters the products as two bf16
// operands, hi = bf16(e) and lo = bf16(e - hi), whose sum is e to about 2^-17
// relative, so the bias keeps binary32 accuracy at two MFMAs per k-step.
template <int NT, bool STAGE, bool EG>  // 32-request tiles per workgroup: 1 or 2; STAGE: coalesced U/G tiles via LDS
__global__ __launch_bounds__(256) void sample_step_mfma(int64_t B, int64_t gamma, int k, int64_t V,
                                                        const bf16_t* __restrict__ U, const bf16_t* __restrict__ W1,
                                                        const bf16_t* __restrict__ W2, const float* __restrict__ G,
                                                        const int32_t* __restrict__ x0,
                                                        const int32_t* __restrict__ force, uint64_t* keys,
                                                        float* __restrict__ logits_out, float* __restrict__ bias_out,
                                                        const float* __restrict__ eg) {
    constexpr int NREQ = 32 * NT;
    constexpr int kEBytes = NREQ * kERow * 2 * (EG ? 2 : 1);
    constexpr int kTileBytes = NREQ * (kURow * 2 + kGRow * 4);
    __shared__ __align__(16) uint8_t lds_raw[kEBytes > kTileBytes ? kEBytes : kTileBytes];
    uint16_t* E_lds = reinterpret_cast<uint16_t*>(lds_raw);
    uint16_t* U_lds = reinterpret_cast<uint16_t*>(lds_raw);                      // after the products
    float* G_lds = reinterpret_cast<float*>(lds_raw + NREQ * kURow * 2);
    __shared__ int32_t xprev[NREQ];
    __shared__ uint64_t wkey[4][NREQ];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 31, half = lane >> 5;
    const int64_t b0 = (int64_t)blockIdx.y * NREQ;
    const int64_t v0 = (int64_t)blockIdx.x * kMfmaRows + wave * 32;

    // Every load below is unconditional from an in-bounds (clamped) address, so
    // the compiler issues them back to back; results of clamped rows or
    // requests are discarded in the epilogue.  Order: the small key loads first
    // (they gate the E gather), then W2, then the U/G tiles.
    const int bl4 = tid >> 2, part = tid & 3;  // 4 threads per request for keys and the E gather
    const bool req_ok = bl4 < NREQ && b0 + bl4 < B;
    const int64_t bq = b0 + (req_ok ? bl4 : 0) < B ? b0 + (req_ok ? bl4 : 0) : B - 1;
    uint64_t kv[kKeyCopies / 4];
    if (k > 0) {
#pragma unroll
        for (int c = 0; c < kKeyCopies / 4; ++c) kv[c] = *key_at(keys, part * (kKeyCopies / 4) + c, gamma, B, k - 1, bq);
    }

    // W2 rows of this wave as A fragments: k-step s takes rank elements
    // 16 s + 8 half .. +7 of row v0 + row (32 contiguous bytes per row per load)
    uint4 a[16];
    {
        const int64_t v = v0 + row < V ? v0 + row : V - 1;
        const uint4* src = reinterpret_cast<const uint4*>(W2 + v * kMfmaRank + half * 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = src[2 * i];
    }

    // U (and G) tiles, issued before the products
    const int64_t vt = (int64_t)blockIdx.x * kMfmaRows;  // first vocabulary row of the tile
    constexpr int UCH = NREQ * kMfmaRows * 2 / 16 / 256;  // 16-byte chunks per thread
    constexpr int GCH = NREQ * kMfmaRows * 4 / 16 / 256;
    u32x4_t us[STAGE ? UCH : 1], gs[STAGE ? GCH : 1];
    float u[STAGE ? 1 : NT][16], gn[STAGE ? 1 : NT][16];
    if constexpr (STAGE) {
#pragma unroll
        for (int i = 0; i < UCH; ++i) {
            const int c = tid + 256 * i, bl = c / 16, col = (c % 16) * 8;
            const int64_t b = b0 + bl < B ? b0 + bl : B - 1;
            const int64_t vc = vt + col < V ? vt + col : V - 8;
            us[i] = *reinterpret_cast<const u32x4_t*>(U + (b * gamma + k) * V + vc);
        }
        if (G) {
#pragma unroll
            for (int i = 0; i < GCH; ++i) {
                const int c = tid + 256 * i, bl = c / 32, col = (c % 32) * 4;
                const int64_t b = b0 + bl < B ? b0 + bl : B - 1;
                const int64_t vc = vt + col < V ? vt + col : V - 4;
                gs[i] = *reinterpret_cast<const u32x4_t*>(G + (b * gamma + k) * V + vc);
            }
        }
    } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t b = b0 + nt * 32 + row < B ? b0 + nt * 32 + row : B - 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t v = v0 + 8 * (r / 4) + 4 * half + (r % 4);
                const int64_t o = (b * gamma + k) * V + (v < V ? v : V - 1);
                u[nt][r] = load_elem(U, o);
                gn[nt][r] = G ? G[o] : 0.f;
            }
        }
    }

    // previous tokens of this workgroup's requests
    {
        int32_t x = -1;
        if (k == 0) {
            x = x0[bq];
        } else {
            uint64_t m = 0;
#pragma unroll
            for (int c = 0; c < kKeyCopies / 4; ++c) m = umax64(m, kv[c]);
            m = umax64(m, shfl_xor_u64(m, 1));
            m = umax64(m, shfl_xor_u64(m, 2));
            const int32_t f = force ? force[bq * gamma + k - 1] : -1;
            x = m == 0 ? -1 : (f >= 0 ? f : key_token(m));
        }
        if (x >= V) x = -1;
        if (bl4 < NREQ && part == 0) xprev[bl4] = req_ok ? (x < 0 ? -1 : x) : -1;
    }
    __syncthreads();
    // gather E = W1[x_prev] (EG: the hi and lo halves of eg) into LDS: 4
    // threads per request, 64 rank elements each
    uint16_t* El_lds = E_lds + NREQ * kERow;  // EG: the lo operand
    if (bl4 < NREQ) {
        const int32_t x = xprev[bl4];
        if constexpr (EG) {
            const float4* src = reinterpret_cast<const float4*>(eg + bq * kMfmaRank + part * 64);
            float4 e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = src[i];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float f[4] = {e[i].x, e[i].y, e[i].z, e[i].w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hi[j] = bf16_rne(f[j]);
                    lo[j] = bf16_rne(f[j] - __uint_as_float(hi[j] << 16));
                }
                const int o = bl4 * kERow + part * 64 + 4 * i;
                *reinterpret_cast<uint2*>(E_lds + o) = make_uint2(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16);
                *reinterpret_cast<uint2*>(El_lds + o) = make_uint2(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16);
            }
        } else {
            const uint4* src = reinterpret_cast<const uint4*>(W1 + (int64_t)(x < 0 ? 0 : x) * kMfmaRank + part * 64);
            uint4 e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = src[i];
            uint4* dst = reinterpret_cast<uint4*>(E_lds + bl4 * kERow + part * 64);
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = e[i];
        }
    }
    __syncthreads();

    f32x16_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a[s]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4 bw = *reinterpret_cast<const uint4*>(E_lds + (nt * 32 + row) * kERow + s * 16 + half * 8);
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bw), acc[nt], 0, 0, 0);
            if constexpr (EG) {
                const uint4 bl = *reinterpret_cast<const uint4*>(El_lds + (nt * 32 + row) * kERow + s * 16 + half * 8);
                acc[nt] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bl), acc[nt], 0, 0, 0);
            }
        }
    }

    if constexpr (STAGE) {  // E is no longer needed: its space takes the U and G tiles
        __syncthreads();
#pragma unroll
        for (int i = 0; i < UCH; ++i) {
            const int c = tid + 256 * i, bl = c / 16, col = (c % 16) * 8;
            *reinterpret_cast<u32x4_t*>(U_lds + bl * kURow + col) = us[i];
        }
        if (G) {
#pragma unroll
            for (int i = 0; i < GCH; ++i) {
                const int c = tid + 256 * i, bl = c / 32, col = (c % 32) * 4;
                *reinterpret_cast<u32x4_t*>(G_lds + bl * kGRow + col) = gs[i];
            }
        }
        __syncthreads();
    }

    // epilogue: lane holds vocabulary rows v0 + 8(r/4) + 4 half + r%4 of request nt*32 + row
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int bl = nt * 32 + row;
        const int64_t b = b0 + bl;
        uint64_t key = 0;
        if (b < B && xprev[bl] >= 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t v = v0 + 8 * (r / 4) + 4 * half + (r % 4);
                if (v < V) {
                    const int vl = wave * 32 + 8 * (r / 4) + 4 * half + (r % 4);  // row within the tile
                    const float uu = STAGE ? widen_lo((uint32_t)U_lds[bl * kURow + vl]) : u[STAGE ? 0 : nt][r];
                    const float gg = !G ? 0.f : (STAGE ? G_lds[bl * kGRow + vl] : gn[STAGE ? 0 : nt][r]);
                    const float bias = acc[nt][r];
                    const float lg = uu + bias;
                    const float sc = G ? lg + gg : lg;
                    const int64_t o = (b * gamma + k) * V + v;
                    if (bias_out) bias_out[o] = bias;
                    if (logits_out) logits_out[o] = lg;
                    key = umax64(key, argmax_key(sc, (uint32_t)v));
                }
            }
        }
        key = umax64(key, shfl_xor_u64(key, 32));
        if (half == 0) wkey[wave][bl] = key;
    }
    __syncthreads();
    if (tid < NREQ && b0 + tid < B) {
        uint64_t m = umax64(umax64(wkey[0][tid], wkey[1][tid]), umax64(wkey[2][tid], wkey[3][tid]));
        if (m != 0)
            atomicMax((unsigned long long*)key_at(keys, (int)(blockIdx.x % kKeyCopies), gamma, B, k, b0 + tid),
                      (unsigned long long)m);
    }
}

// ---------------------------------------------------------------------------
// Batched sampler with W2 resident on the matrix cores (bf16, rank 256,
// 16..64 requests).
//
// One persistent workgroup per CU, eight waves.  Workgroup g owns a
// contiguous range of up to 20 32-row vocabulary tiles of W2 for the whole
// block: wave w holds tiles t0 + w and t0 + w + 8 in registers as
// v_mfma_f32_32x32x16_bf16 A fragments, and tiles t0 + 16 .. t0 + 19 sit in
// LDS (rows padded against bank conflicts), one per wave 0..3.  W2 crosses
// HBM once per call and a step streams only U (and G).
// Step k: gather E = W1[x_{k-1}] of every request into LDS (the B operand),
// multiply each held tile by it, fuse + U (+ G) and the argmax in the
// accumulator layout (one request per lane, 16 rows in-lane), reduce over
// the waves, and publish one packed key per request.  Workgroup r < B
// reduces request r over all workgroups and posts the winner in 8 copies of
// the 64-word winner array; workgroup g reads copy g % 8 for step k + 1.  Workgroup 0 computes the
// confidence and the running survival of every request per step.  Every
// exchanged word is self-validating (never zero when written) and is
// cleared one step later by its writer, when all its readers are provably
// past it; the last step's words go to the last workgroup out.
// ---------------------------------------------------------------------------
constexpr int kResRegTiles = 2;  // 32-row W2 tiles held in registers per wave
constexpr int kResWaves = 8;
constexpr int kResLdsTiles = 3;  // more tiles per workgroup held in LDS
constexpr int kResThreads = 64 * kResWaves;
constexpr int kResMaxTiles = kResWaves * kResRegTiles + kResLdsTiles;
constexpr int kResMaxReq = 64;
constexpr int kResCopies = 8;   // copies of the winner words
constexpr int kResMaxWGs = 256;
constexpr size_t kResHeader = kWsHeader;  // words 0 (exit counter), 1 (status), 3 (paths)
constexpr int kResMaxGamma = 8;  // block width of the gated and RNN heads in this kernel

__device__ __forceinline__ int32_t winner_token(uint64_t key) {  // 0 or 1: no candidate
    return key <= 1 ? -1 : key_token(key);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Read back one 32 x 32 Gumbel unit that buffer_load_dwordx4 ... lds put into
// LDS (lane l's 16 bytes of load c at c * 1024 + 16 l).  The compiler does
// not tell apart the LDS slots those loads fill and would wait for every
// load in flight before any read of them, so the read is written out here.
// The U words of the same unit are passed in only as a dependency: they were
// loaded after this unit's Gumbel loads, and vector memory loads complete in
// order, so the wait the compiler puts in front for them also covers the
// Gumbel data.  The trailing wait makes the slot free for its next load.
// There is no memory clobber, which would make the compiler wait for every
// LDS load in flight, the next unit's included; callers fence the read with
// scheduling barriers instead.
__device__ __forceinline__ void read_gumbel_unit(uint32_t lds_addr, const u32x4_t (&dep)[2], f32x4_t (&g)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(g[0]), "=&v"(g[1]), "=&v"(g[2]), "=&v"(g[3])
        : "v"(lds_addr), "v"(dep[0]), "v"(dep[1]));
}

// HD: the sequential head.  0: the Markov head (E = W1[x_{k-1}]).  1: the
// gated head and 2: the RNN head, whose binary32 embedding enters the
// products as hi and lo bf16 halves (see sample_step_mfma).  With HD != 0,
// workgroup g < r computes column j = g of every request's embedding per
// step and posts it as tagged words; every workgroup then reads all columns
// back.  Wh, Wh2: Wg, or Wrg and Wrc; hid: their hidden halves as hks
// split-K partials of [B][gamma][r] each (Wrg's, then Wrc's for the RNN
// head); ebw: the posted columns, two step slots of [64][r] words.  HD != 0
// needs NT == 2, at least r workgroups and gamma <= kResMaxGamma.
template <int NT, bool HG, int HD>
__global__ __launch_bounds__(kResThreads) void sample_batch_resident(int64_t B, int gamma, int64_t V, int tiles_per_wg, const bf16_t* __restrict__ U,
                      const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W2, const bf16_t* __restrict__ h,
                      const bf16_t* __restrict__ w_conf, int64_t H, float b_conf, const int32_t* __restrict__ x0,
                      const float* __restrict__ G, const int32_t* __restrict__ force, int32_t* __restrict__ tokens,
                      float* __restrict__ conf, float* __restrict__ survival, uint64_t* hword, uint64_t* pub,
                      uint64_t* win, uint32_t* header, int spin_limit, const bf16_t* __restrict__ Wh,
                      const bf16_t* __restrict__ Wh2, float* __restrict__ hid, int hks, uint64_t* ebw) {
    constexpr int NREQ = 32 * NT;
    constexpr bool EG = HD != 0;
    static_assert(!EG || NT == 2, "the gated and RNN heads run with two request blocks");
    // the hi and lo halves need a second E; with Gumbel noise that space
    // comes from a single Gumbel slot per wave
    constexpr int kGSlots = (EG && HG) ? 1 : 2;
    __shared__ __align__(16) uint16_t E_lds[NREQ * kERow * (EG ? 2 : 1)];
    uint16_t* const El_lds = E_lds + (EG ? NREQ * kERow : 0);  // EG: the lo halves
    __shared__ __align__(16) uint16_t T_lds[kResLdsTiles * 32 * kERow];  // W2 tiles held in LDS
    __shared__ __align__(16) float G_lds[kResWaves][kGSlots][32 * 32];  // per wave: Gumbel units in flight
    // EG: this workgroup's row of the head weights as bf16 pairs (gated: the
    // embedding half of Wg; RNN: the state and embedding halves of Wrg, then
    // of Wrc), and for the RNN head its column of the state and the state
    // halves of the next step's two products
    constexpr int kHWords = HD == 2 ? 2 * kMfmaRank : (HD == 1 ? kMfmaRank / 2 : 1);
    __shared__ uint32_t hrow[kHWords];
    __shared__ float zs_lds[2][HD == 2 ? NREQ : 1];
    __shared__ float s_lds[HD == 2 ? NREQ : 1];
    // EG: the hidden halves of column g for every request and step (gated:
    // Wg's; RNN: Wrg's then Wrc's), read once at the start
    __shared__ float hcol[EG ? HD * kResMaxReq * kResMaxGamma : 1];
    __shared__ uint64_t wkey[kResWaves][NREQ];
    __shared__ uint64_t rkey[kResWaves];
    __shared__ int rlost[kResWaves];
    __shared__ int32_t xprev[NREQ];
    __shared__ uint32_t we_lds[kMfmaRank / 2];  // Markov part of the confidence weights (workgroup 0)
    __shared__ int last_flag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 31, half = lane >> 5;
    const int g = blockIdx.x, nwg = gridDim.x;
    const int64_t ntiles = (V + 31) / 32;
    const int64_t t0 = (int64_t)g * tiles_per_wg;
    const int64_t t_end = t0 + tiles_per_wg < ntiles ? t0 + tiles_per_wg : ntiles;
    const uint64_t* wcopy = win + (int64_t)(g % kResCopies) * kResMaxReq;  // step stride kResCopies * 64
    if (g == 0 && tid == 0) mark_path(header, kPathResident);

    // this wave's W2 tiles, as A fragments: k-step s holds rank elements
    // 16 s + 8 half .. +7 of row 32 t + row
    uint4 a[kResRegTiles][16];
#pragma unroll
    for (int i = 0; i < kResRegTiles; ++i) {
        const int64_t t = t0 + wave + kResWaves * i;
        int64_t v = t * 32 + row;
        v = (t < t_end && v < V) ? v : 0;  // clamped; its products are never used
        const uint4* src = reinterpret_cast<const uint4*>(W2 + v * kMfmaRank + half * 8);
#pragma unroll
        for (int s = 0; s < 16; ++s) a[i][s] = src[2 * s];
    }
    // the LDS tiles: 16 bytes per thread per pass, 4 passes cover 4 x 32 rows
#pragma unroll
    for (int pss = 0; pss < kResLdsTiles * 32 * 32 / kResThreads; ++pss) {
        const int c = tid + kResThreads * pss;  // 16-byte chunk: row c / 32 of the 128, column (c % 32) * 8
        const int lr = c / 32, col = (c % 32) * 8;
        const int64_t t = t0 + kResWaves * kResRegTiles + lr / 32;
        int64_t v = t * 32 + lr % 32;
        v = (t < t_end && v < V) ? v : 0;
        *reinterpret_cast<uint4*>(T_lds + lr * kERow + col) =
            *reinterpret_cast<const uint4*>(W2 + v * kMfmaRank + col);
    }

    if (g == 0 && tid < kMfmaRank / 2)
        we_lds[tid] = (uint32_t)w_conf[H + 2 * tid].bits | ((uint32_t)w_conf[H + 2 * tid + 1].bits << 16);
    if constexpr (HD == 1) {
        if (g < kMfmaRank && tid < kMfmaRank / 2) {
            const bf16_t* wr = Wh + (int64_t)g * (H + kMfmaRank) + H + 2 * tid;
            hrow[tid] = (uint32_t)wr[0].bits | ((uint32_t)wr[1].bits << 16);
        }
    }
    if constexpr (HD == 2) {
        if (g < kMfmaRank) {  // kResThreads == 2 r: one pair per thread
            const bf16_t* wr = (tid < kMfmaRank ? Wh : Wh2) + (int64_t)g * (2 * kMfmaRank + H) + 2 * (tid % kMfmaRank);
            hrow[tid] = (uint32_t)wr[0].bits | ((uint32_t)wr[1].bits << 16);
        }
        if (tid < NREQ) zs_lds[0][tid] = zs_lds[1][tid] = s_lds[tid] = 0.f;  // s_0 = 0
    }
    if constexpr (EG) {
        // this workgroup's column of the hidden halves, which no other
        // workgroup reads: it zeroes the words once they are loaded
        if (g < kMfmaRank) {
            // column-major halves: the column is B gamma contiguous floats per range
            const int64_t mr = B * gamma * kMfmaRank;
            for (int i = tid; i < HD * B * gamma; i += kResThreads) {  // i = (m B + b) gamma + k
                const int64_t m = i / (B * gamma), bk = i % (B * gamma);
                float v = 0.f;
                for (int ks = 0; ks < hks; ++ks) v += hid[(m * hks + ks) * mr + g * B * gamma + bk];
                hcol[i] = v;
                for (int ks = 0; ks < hks; ++ks) hid[(m * hks + ks) * mr + g * B * gamma + bk] = 0.f;
            }
        }
    }
    // a wave's work per step is a list of units (tile i, 32-request block nt),
    // unit p = i * NT + nt; the tiles it holds form a prefix of register
    // tile 0, register tile 1, LDS tile
    constexpr int kUnits = (kResRegTiles + 1) * NT;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int ntw = 0;
    if (t0 + wv < t_end) ntw = 1;
    if (t0 + wv + kResWaves < t_end) ntw = 2;
    if (wv < kResLdsTiles && t0 + kResWaves * kResRegTiles + wv < t_end) ntw = 3;
    const int n_units = ntw * NT;
    // U of unit p lives in uq[p % 2], its Gumbel values in G_lds[wave][p % 2].
    // issue(slot, u, kk) starts the loads of unit u of step kk into that slot;
    // u < 0 is a stand-in (every lane loads the first element group, a cache
    // hit) so that every path through the unit loop has the same loads in
    // flight and the waits the compiler places stay at unit depth
    // Lane (row, half) loads the U rows vt + 16 i + 8 half .. + 7 (i = 0, 1)
    // as two 16-byte pieces, so the two lanes of a request read 32
    // contiguous bytes per instruction; the epilogue's rows
    // vt + 8 c + 4 half .. + 3 are then one swap of 8-byte halves between
    // lanes l and l + 32 away (unit_u).
    u32x4_t uq[2][2];
    // the Gumbel loads go through a buffer descriptor (the caller keeps G
    // under 2 GiB): the global_load_lds form makes the compiler wait for all
    // vector memory loads at every later wait, the buffer form does not
    const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(G), (short)0, (int)(B * gamma * V * 4), 0x00020000);
    auto issue = [&](const int slot, const int u, const int kk) {
        __builtin_amdgcn_sched_barrier(0);
        const bool real = u >= 0;
        const int uu = real ? u : 0;
        const int i = uu / NT, nt = uu % NT;
        const int64_t t = i < kResRegTiles ? t0 + wv + kResWaves * i : t0 + kResWaves * kResRegTiles + wv;
        const int bl = nt * 32 + row;
        const int64_t base = real ? ((int64_t)(bl < B ? bl : B - 1) * gamma + kk) * V : 0;
        // first row of the tile, opaque to the optimiser: the addresses are
        // cheap to recompute, and hoisting them out of the step loop spills
        int vt = (int)(t * 32);
        asm volatile("" : "+v"(vt));
        int64_t v[4], vu[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t x = vt + 8 * c + 4 * half;
            v[c] = !real ? 0 : x + 4 <= V ? x : V - 4;  // clamped (V is a multiple of 8); masked in the epilogue
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t x = vt + 16 * i + 8 * half;
            vu[i] = !real ? 0 : x + 8 <= V ? x : V - 8;
        }
        if constexpr (HG) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(g_rsrc, (lds_void_t*)&G_lds[wv][kGSlots == 1 ? 0 : slot][c * 256], 16,
                                                         (uint32_t)(base + v[c]) * 4u, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // U strictly after this unit's Gumbel loads
#pragma unroll
        for (int i = 0; i < 2; ++i) uq[slot][i] = *reinterpret_cast<const u32x4_t*>(U + base + vu[i]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // The lane's epilogue rows from the unit's two pieces, in place: after
    // swapping the high 8 bytes of lanes 0-31 with the low 8 bytes of lanes
    // 32-63, piece i's low half holds rows 16 i + 4 half .. + 3 and its high
    // half rows 16 i + 8 + 4 half .. + 3 in every lane, so rows
    // 8 c + 4 half .. + 3 are words 2 (c % 2), + 1 of piece c / 2.
    auto unit_u = [&](const int slot) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(uq[slot][i][0], uq[slot][i][2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(uq[slot][i][1], uq[slot][i][3], false, false);
            uq[slot][i] = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
        }
    };
    issue(0, 0 < n_units ? 0 : -1, 0);
    if constexpr (kGSlots == 2) issue(1, 1 < n_units ? 1 : -1, 0);

    // the hidden part of every confidence logit, w_h . h[b, k]: pair
    // p = b gamma + k goes to wave p of the grid and is posted as a tagged
    // word that workgroup 0 reads at step k.  No barrier here, so these loads
    // overlap the W2 loads above.
    for (int64_t p = (int64_t)g * kResWaves + wv; p < B * gamma; p += (int64_t)nwg * kResWaves) {  // wave-uniform
        const bf16_t* hr = h + p * H;
        float hs = 0.f;
        if (H % 8 == 0 && (uintptr_t)h % 16 == 0 && (uintptr_t)w_conf % 16 == 0) {
            const uint4* hv = reinterpret_cast<const uint4*>(hr);
            const uint4* cv = reinterpret_cast<const uint4*>(w_conf);
            const int64_t n = H / 8;
            for (int64_t i0 = lane; i0 < n; i0 += 64 * 8) {
                uint4 a[8], c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t i = i0 + 64 * j < n ? i0 + 64 * j : 0;  // clamped; masked below
                    a[j] = hv[i];
                    c[j] = cv[i];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i0 + 64 * j < n)
                        hs = dot2(c[j].w, a[j].w, dot2(c[j].z, a[j].z, dot2(c[j].y, a[j].y, dot2(c[j].x, a[j].x, hs))));
            }
        } else {
            for (int64_t i = lane; i < H; i += 64) hs += load_elem(w_conf, i) * load_elem(hr, i);
        }
        for (int o = 32; o > 0; o >>= 1) hs += __shfl_xor(hs, o);
        if (lane == 0)
            __hip_atomic_store(hword + p, kTag | __float_as_uint(hs), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    float A = 1.f;  // workgroup 0, thread 4 b: running survival of request b
    for (int k = 0; k < gamma; ++k) {

        // previous tokens: the anchors, then the winners of the last step
        if (tid < NREQ) {
            int64_t x = -1;
            if (tid < B) {
                if (k == 0) {
                    x = x0[tid];
                } else {
                    const uint64_t* p = wcopy + (int64_t)(k - 1) * kResCopies * kResMaxReq + tid;
                    uint64_t w = 0;
                    for (int spin = 0; spin < spin_limit && w == 0; ++spin) {
                        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (w == 0) __builtin_amdgcn_s_sleep(1);
                    }
                    if (w == 0) mark_gave_up(header);  // timed out: reported as token -1
                    const int32_t tok = winner_token(w);
                    const int32_t f = (force && tok >= 0) ? force[tid * gamma + k - 1] : -1;
                    x = tok < 0 ? -1 : (f >= 0 ? f : tok);
                }
            }
            xprev[tid] = (x >= 0 && x < V) ? (int32_t)x : -1;
            // every reducer has read this workgroup's keys of the last step
            if (k > 0 && tid < B)
                __hip_atomic_store(pub + ((int64_t)(k - 1) * nwg + g) * kResMaxReq + tid, (uint64_t)0,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        // gather E = W1[x_prev] into LDS: 4 threads per request, 128 bytes each
        {
            const int bl = tid >> 2, part = tid & 3;
            if (bl < NREQ) {
                const int32_t x = xprev[bl];
                const uint4* src = reinterpret_cast<const uint4*>(W1 + (int64_t)(x < 0 ? 0 : x) * kMfmaRank + part * 64);
                uint4 e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = src[i];
                uint4* dst = reinterpret_cast<uint4*>(E_lds + bl * kERow + part * 64);
#pragma unroll
                for (int i = 0; i < 8; ++i) dst[i] = e[i];
            }
        }
        __syncthreads();
        // workgroup 0: confidence and survival of step k (its Markov part needs e)
        if (g == 0) {
            const int bl = tid >> 2, part = tid & 3;
            if (bl < NREQ) {
                const uint32_t* er = reinterpret_cast<const uint32_t*>(E_lds + bl * kERow + part * 64);
                float s = 0.f;
#pragma unroll 8
                for (int q = 0; q < 32; ++q) s = dot2(we_lds[part * 32 + q], er[q], s);
                s += __shfl_xor(s, 1);
                s += __shfl_xor(s, 2);
                if (part == 0 && bl < B) {
                    const bool live = xprev[bl] >= 0;
                    uint64_t hw = 0;  // posted in the prologue, normally long before
                    for (int spin = 0; spin < spin_limit && hw == 0; ++spin) {
                        hw = __hip_atomic_load(hword + bl * gamma + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (hw == 0) __builtin_amdgcn_s_sleep(1);
                    }
                    if (hw == 0) mark_gave_up(header);  // reported as NaN confidence
                    const float hd = hw != 0 ? __uint_as_float((uint32_t)hw) : __builtin_nanf("");
                    const float c = 1.f / (1.f + expf(-(hd + s + b_conf)));
                    A = A * c;
                    conf[bl * gamma + k] = live ? c : __builtin_nanf("");
                    survival[bl * gamma + k] = live ? A : __builtin_nanf("");
                }
            }
        }

        if constexpr (EG) {
            // the head's embedding.  Column j = g of every request, from the
            // bf16 rows e = W1[x_{k-1}] in E (8 threads per request, 32 rank
            // elements each), posted as a word tagged with the step
            const int bl = tid >> 3, part = tid & 7;
            if (g < kMfmaRank) {
                const uint32_t* er = reinterpret_cast<const uint32_t*>(E_lds + bl * kERow + part * 32);
                float d1 = 0.f, d2 = 0.f;  // embedding halves of the products with this row
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const uint32_t ev = er[q];
                    if constexpr (HD == 1) {
                        d1 = dot2(hrow[part * 16 + q], ev, d1);
                    } else {
                        d1 = dot2(hrow[kMfmaRank / 2 + part * 16 + q], ev, d1);
                        d2 = dot2(hrow[kMfmaRank + kMfmaRank / 2 + part * 16 + q], ev, d2);
                    }
                }
                d1 += __shfl_xor(d1, 1);
                d1 += __shfl_xor(d1, 2);
                d1 += __shfl_xor(d1, 4);
                if constexpr (HD == 2) {
                    d2 += __shfl_xor(d2, 1);
                    d2 += __shfl_xor(d2, 2);
                    d2 += __shfl_xor(d2, 4);
                }
                if (part == 0) {  // requests past B: any finite column
                    const int64_t bk = (int64_t)(bl < B ? bl : B - 1) * gamma + k;
                    const float hg = hcol[bk];
                    float val;
                    if constexpr (HD == 1) {
                        // eb_j = e_j sigmoid(Wg[j] . [h_k; e])
                        const float ej = __uint_as_float((uint32_t)E_lds[bl * kERow + g] << 16);
                        val = ej / (1.f + expf(-(hg + d1)));
                    } else {
                        // s_k[j] = u s_{k-1}[j] + (1 - u) tanh(Wrc[j] . z), u = sigmoid(Wrg[j] . z)
                        const float zg = hg + zs_lds[0][bl] + d1;
                        const float zc = hcol[B * gamma + bk] + zs_lds[1][bl] + d2;
                        const float u = 1.f / (1.f + expf(-zg));
                        val = u * s_lds[bl] + (1.f - u) * tanhf(zc);
                        s_lds[bl] = val;
                    }
                    __hip_atomic_store(ebw + ((int64_t)(k & 1) * kResMaxReq + bl) * kMfmaRank + g,
                                       ((uint64_t)(k + 1) << 32) | __float_as_uint(val), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();  // E's bf16 rows are read: their space takes the hi halves
            // every column comes back as the hi and lo bf16 halves of E: wave w
            // reads requests 8 w .. 8 w + 7, lane l columns 2 l, 2 l + 1 and
            // 128 + 2 l, 129 + 2 l of each (consecutive lanes, consecutive
            // words), in two runs of four requests with all their loads in
            // flight.  The RNN head also forms the state halves of the next
            // step's two products, one wave sum per request.
            {
                const uint64_t* src = ebw + (int64_t)(k & 1) * kResMaxReq * kMfmaRank;
                const uint32_t want = (uint32_t)(k + 1);
                const int wvr = __builtin_amdgcn_readfirstlane(wave);
                bool all = true;
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    uint64_t w[16];  // request q of the run, column c: w[4 q + c]
                    auto addr = [&](int i) {
                        const int q = i >> 2, c = i & 3;
                        const int col = (c < 2 ? 0 : kMfmaRank / 2) + 2 * lane + (c & 1);
                        return src + (int64_t)(wvr * 8 + run * 4 + q) * kMfmaRank + col;
                    };
#pragma unroll
                    for (int i = 0; i < 16; ++i) w[i] = __hip_atomic_load(addr(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    bool ok = true;
#pragma unroll
                    for (int i = 0; i < 16; ++i) ok = ok && (uint32_t)(w[i] >> 32) == want;
                    for (int spin = 0; !__all(ok) && spin < spin_limit; ++spin) {
                        __builtin_amdgcn_s_sleep(1);
                        ok = true;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            if ((uint32_t)(w[i] >> 32) != want)
                                w[i] = __hip_atomic_load(addr(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            ok = ok && (uint32_t)(w[i] >> 32) == want;
                        }
                    }
                    all = all && __all(ok);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int bq = wvr * 8 + run * 4 + q;
                        float zg = 0.f, zc = 0.f;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {  // columns 2 l (+ 128), and the next
                            const float f0 = __uint_as_float((uint32_t)w[4 * q + 2 * hh]);
                            const float f1 = __uint_as_float((uint32_t)w[4 * q + 2 * hh + 1]);
                            const uint32_t h0 = bf16_rne(f0), h1 = bf16_rne(f1);
                            const uint32_t l0 = bf16_rne(f0 - __uint_as_float(h0 << 16));
                            const uint32_t l1 = bf16_rne(f1 - __uint_as_float(h1 << 16));
                            const int o = bq * kERow + hh * (kMfmaRank / 2) + 2 * lane;
                            *reinterpret_cast<uint32_t*>(E_lds + o) = (h0 & 0xffffu) | (h1 << 16);
                            *reinterpret_cast<uint32_t*>(El_lds + o) = (l0 & 0xffffu) | (l1 << 16);
                            if constexpr (HD == 2) {
                                const int pr = hh * (kMfmaRank / 4) + lane;  // state-half pair of Wrg / Wrc
                                zg = __builtin_fmaf(widen_hi(hrow[pr]), f1, __builtin_fmaf(widen_lo(hrow[pr]), f0, zg));
                                zc = __builtin_fmaf(widen_hi(hrow[kMfmaRank + pr]), f1,
                                                    __builtin_fmaf(widen_lo(hrow[kMfmaRank + pr]), f0, zc));
                            }
                        }
                        if constexpr (HD == 2) {
                            zg = wave_sum_f32(zg);
                            zc = wave_sum_f32(zc);
                            if (lane == 0) zs_lds[0][bq] = zg, zs_lds[1][bq] = zc;
                        }
                    }
                }
                if (!all && lane == 0) mark_gave_up(header);  // a column never came: the step's tokens are unspecified
            }
            __syncthreads();
        }

        // the products, the + U (+ G) epilogue and the in-lane argmax, one unit
        // at a time with the U and Gumbel loads of the unit after next in flight
        // (with one Gumbel slot, of the next unit)
        uint64_t key[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) key[nt] = 0;
#pragma unroll
        for (int p = 0; p < kUnits; ++p) {
            if (p >= n_units) break;  // wave-uniform; the units held form a prefix
            const int i = p / NT, nt = p % NT;
            const bool lds_tile = i == kResRegTiles;
            const int64_t t = lds_tile ? t0 + kResWaves * kResRegTiles + wv : t0 + wv + kResWaves * i;
            __builtin_amdgcn_sched_barrier(0);
            f32x16_t acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const uint4 aw = lds_tile ? *reinterpret_cast<const uint4*>(T_lds + (wv * 32 + row) * kERow + s * 16 + half * 8)
                                          : a[i < kResRegTiles ? i : 0][s];
                const uint4 bw = *reinterpret_cast<const uint4*>(E_lds + (nt * 32 + row) * kERow + s * 16 + half * 8);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                              __builtin_bit_cast(bf16x8_t, bw), acc, 0, 0, 0);
                if constexpr (EG) {
                    const uint4 bw2 = *reinterpret_cast<const uint4*>(El_lds + (nt * 32 + row) * kERow + s * 16 + half * 8);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                                  __builtin_bit_cast(bf16x8_t, bw2), acc, 0, 0, 0);
                }
            }
            unit_u(p & 1);
            f32x4_t gr[4];
            if constexpr (HG) {
                const uint32_t ga = (uint32_t)(uintptr_t)(lds_void_t*)&G_lds[wv][kGSlots == 1 ? 0 : (p & 1)][lane * 4];
                __builtin_amdgcn_sched_barrier(0);
                read_gumbel_unit(ga, uq[p & 1], gr);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kGSlots == 1) {
                // the one Gumbel slot is free: the next unit's loads (after the
                // last unit, the next step's first; the unit count is even)
                const bool last = p + 1 >= n_units;
                issue((p + 1) & 1, last ? (k + 1 < gamma ? 0 : -1) : p + 1, last ? k + 1 : k);
            }
            const int bl = nt * 32 + row;
            if (bl < B && xprev[bl] >= 0) {
                int vt = (int)(t * 32);
                asm volatile("" : "+v"(vt));
                // lane element r is row vt + 8 (r / 4) + 4 half + r % 4: rows rise with r
                auto score = [&](const int r, float& bias, float& lg) {
                    const int c = r / 4, q = r % 4;
                    const uint32_t uw = uq[p & 1][c >> 1][2 * (c & 1) + (q >> 1)];
                    bias = acc[r];
                    lg = ((q & 1) ? widen_hi(uw) : widen_lo(uw)) + bias;
                    if constexpr (HG) return lg + gr[c][q];
                    return lg;
                };
                if (vt + 32 <= V) {  // wave-uniform
                    // whole tile in range: first maximum in float compares, one
                    // packed key per unit (+ 0 maps -0 onto +0)
                    float bias, lg;
                    float best = score(0, bias, lg);
                    int bi = 0;
#pragma unroll
                    for (int r = 1; r < 16; ++r) {
                        const float sc = score(r, bias, lg);
                        if (sc > best) {
                            best = sc;
                            bi = r;
                        }
                    }
                    const uint32_t v = (uint32_t)(vt + 8 * (bi >> 2) + 4 * half + (bi & 3));
                    key[nt] = umax64(key[nt], argmax_key(best + 0.f, v));
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t v = vt + 8 * (r / 4) + 4 * half + r % 4;
                        if (v >= V) continue;
                        float bias, lg;
                        const float sc = score(r, bias, lg);
                        key[nt] = umax64(key[nt], argmax_key(sc + 0.f, (uint32_t)v));
                    }
                }
            }
            if constexpr (kGSlots == 2) issue(p & 1, p + 2 < n_units ? p + 2 : -1, k);
        }
        // the first two units of the next step need nothing from this one
        if (kGSlots == 2 && k + 1 < gamma) {
            issue(0, 0 < n_units ? 0 : -1, k + 1);
            issue(1, 1 < n_units ? 1 : -1, k + 1);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            key[nt] = umax64(key[nt], shfl_xor_u64(key[nt], 32));
            if (half == 0) wkey[wave][nt * 32 + row] = key[nt];
        }
        __syncthreads();
        // publish this workgroup's best key per request (1 = no candidate)
        if (tid < B) {
            uint64_t m = 0;
#pragma unroll
            for (int w = 0; w < kResWaves; ++w) m = umax64(m, wkey[w][tid]);
            __hip_atomic_store(pub + ((int64_t)k * nwg + g) * kResMaxReq + tid, m ? m : 1ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        // workgroup g reduces requests g, g + nwg, ... over every workgroup
        for (int r = g; r < B; r += nwg) {  // workgroup-uniform
            uint64_t m = 0;
            if (tid < nwg) {
                const uint64_t* p = pub + ((int64_t)k * nwg + tid) * kResMaxReq + r;
                for (int spin = 0; spin < spin_limit && m == 0; ++spin) {
                    m = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (m == 0) __builtin_amdgcn_s_sleep(1);
                }
            }
            // a workgroup whose key never arrived leaves the step without a
            // winner (token -1), not with the best of the others
            const bool lost = __any(tid < nwg && m == 0);
            m = wave_max_u64(m);
            if (lane == 0) rkey[wave] = m, rlost[wave] = lost ? 1 : 0;
            __syncthreads();
            uint64_t best = 0;
            bool missing = false;
#pragma unroll
            for (int w = 0; w < kResWaves; ++w) missing = missing || rlost[w] != 0, best = umax64(best, rkey[w]);
            if (missing) best = 0;
            if (missing && tid == 0) mark_gave_up(header);
            if (tid < kResCopies)
                __hip_atomic_store(win + ((int64_t)k * kResCopies + tid) * kResMaxReq + r, best ? best : 1ull,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) tokens[r * gamma + k] = winner_token(best);
            // every workgroup has read the winners of the last step: they
            // published this step's keys after it
            if (k > 0 && tid >= 64 && tid < 64 + kResCopies)
                __hip_atomic_store(win + ((int64_t)(k - 1) * kResCopies + (tid - 64)) * kResMaxReq + r, (uint64_t)0,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (EG) {
                // after the last step's keys every workgroup is past its last
                // read of the posted columns: request r's words of both step
                // slots are cleared here, and those of padding row r + B if
                // there is one (every row up to kResMaxReq is posted; B > 32
                // gives each padding row one reducer).  After a give-up a late
                // workgroup may still post; the last one out clears everything
                // then.
                if (k == gamma - 1 && !missing) {
                    const int nrow = r + B < kResMaxReq ? 2 : 1;
                    for (int i = tid; i < nrow * 2 * kMfmaRank; i += kResThreads) {
                        const int row = i < 2 * kMfmaRank ? r : r + (int)B, j = i % (2 * kMfmaRank);
                        __hip_atomic_store(ebw + ((int64_t)(j / kMfmaRank) * kResMaxReq + row) * kMfmaRank +
                                               j % kMfmaRank,
                                           (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            __syncthreads();  // rkey is reused
        }
        __syncthreads();  // wkey and rkey are reused next step
    }

    // leave: the last workgroup out clears the last step's words
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&header[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == (uint32_t)(nwg - 1);
    }
    __syncthreads();
    if (last_flag) {
        const int64_t k = gamma - 1;
        for (int64_t i = tid; i < (int64_t)nwg * kResMaxReq; i += kResThreads)
            __hip_atomic_store(pub + k * nwg * kResMaxReq + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = tid; i < kResCopies * kResMaxReq; i += kResThreads)
            __hip_atomic_store(win + k * kResCopies * kResMaxReq + i, (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        for (int64_t i = tid; i < B * gamma; i += kResThreads)
            __hip_atomic_store(hword + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (EG) {  // after a give-up: both step slots of the posted columns
            if (__hip_atomic_load(header + kHdrStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                for (int i = tid; i < 2 * kResMaxReq * kMfmaRank; i += kResThreads)
                    __hip_atomic_store(ebw + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) __hip_atomic_store(&header[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

struct ResidentPlan {
    int nwg = 0, tiles_per_wg = 0;
};

ResidentPlan resident_plan(int64_t B, int64_t V, int hd = 0) {
    ResidentPlan p;
    const int cus = device_cus();
    if (cus <= 0 || B < kMfmaMinBatch || B > kResMaxReq || V % 8 != 0) return p;
    int64_t nwg = cus < kResMaxWGs ? cus : kResMaxWGs;
    const int64_t ntiles = (V + 31) / 32;
    if (nwg > ntiles) nwg = ntiles;
    const int64_t per = (ntiles + nwg - 1) / nwg;
    if (per > (int64_t)kResMaxTiles) return p;
    int per_cu = 0;
    // the Gumbel variants use the most LDS and registers
    const void* fn = hd == 1   ? reinterpret_cast<const void*>(&sample_batch_resident<2, true, 1>)
                     : hd == 2 ? reinterpret_cast<const void*>(&sample_batch_resident<2, true, 2>)
                     : B <= 32 ? reinterpret_cast<const void*>(&sample_batch_resident<1, true, 0>)
                               : reinterpret_cast<const void*>(&sample_batch_resident<2, true, 0>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kResThreads, 0) != hipSuccess || per_cu < 1)
        return p;
    p.nwg = (int)nwg;
    p.tiles_per_wg = (int)per;
    return p;
}

size_t resident_workspace(int64_t B, int64_t gamma) {
    return kResHeader + ((size_t)(8 * B * gamma) + 255) / 256 * 256 +
           (size_t)8 * gamma * kResMaxWGs * kResMaxReq + (size_t)8 * gamma * kResCopies * kResMaxReq;
}

// the gated (hd 1) or RNN (hd 2) head in the resident kernel: its hidden
// halves ([B][gamma][r] floats, two sets for the RNN head) and the posted
// columns (two step slots of [64][r] words) follow the resident words
size_t resident_head_workspace(int64_t B, int64_t gamma, int hd) {
    return resident_workspace(B, gamma) + ((size_t)(4 * hd * kHidMaxSplits * B * gamma * kMfmaRank) + 255) / 256 * 256 +
           (size_t)8 * 2 * kResMaxReq * kMfmaRank;
}

struct Buffers {
    uint64_t* keys;
    float* hdot;
};

Buffers carve(void* ws, int64_t B, int64_t gamma, int ncopy) {
    char* p = static_cast<char*>(ws) + kWsHeader;
    Buffers s;
    s.keys = reinterpret_cast<uint64_t*>(p);
    p += ((size_t)(8 * kKeyStride * ncopy * B * gamma) + 255) / 256 * 256;
    s.hdot = reinterpret_cast<float*>(p);
    return s;
}

template <typename T, int BG>
hipError_t launch_steps(int lpr, int64_t B, int64_t gamma, int k, int64_t V, int64_t r, const T* U, const T* W1,
                        const T* W2, const float* G, const int32_t* x0, const int32_t* force, uint64_t* keys,
                        float* lo, float* bo, const float* eg, hipStream_t stream) {
    const dim3 grid((uint32_t)((V + kTile - 1) / kTile), (uint32_t)((B + BG - 1) / BG));
    const size_t shm = sizeof(float) * BG * r;
#define DSPARK_STEP(L)                                                                                           \
    hipLaunchKernelGGL((sample_step<T, BG, L>), grid, dim3(kThreads), shm, stream, B, gamma, k, V, r, U, W1, W2, \
                       G, x0, force, keys, lo, bo, eg)
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

bool chain_eligible(int64_t B, int64_t r, int dtype, const void* W1, const void* W2) {
    return B == 1 && r == kChainRank && dtype == kBF16 && ((uintptr_t)W1 % 16 == 0) && ((uintptr_t)W2 % 16 == 0);
}

template <typename T>
hipError_t launch_typed(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, const void* U, const void* h,
                        const void* W1, const void* W2, const void* w_conf, float b_conf, const int32_t* x0,
                        const float* G, const int32_t* force, int32_t* tokens, float* conf, float* survival,
                        float* lo, float* bo, void* ws, hipStream_t stream, const void* Wg, const void* Wrg,
                        const void* Wrc) {
    const T* Ut = static_cast<const T*>(U);
    const T* W1t = static_cast<const T*>(W1);
    const T* W2t = static_cast<const T*>(W2);
    const T* wt = static_cast<const T*>(w_conf);

    // batched bf16 rank-256 requests go to the matrix cores (a gated or RNN
    // head reads its binary32 embeddings from the workspace with 16-byte loads)
    const bool headed = Wg != nullptr || Wrg != nullptr;
    bool mfma = false;
    if constexpr (std::is_same_v<T, bf16_t>)
        mfma = r == kMfmaRank && B >= kMfmaMinBatch && ((uintptr_t)W1 % 16 == 0) && ((uintptr_t)W2 % 16 == 0) &&
               (!headed || (uintptr_t)ws % 16 == 0);
    if constexpr (std::is_same_v<T, bf16_t>) {
        // resident W2: one persistent kernel for the whole block.  The gated
        // and RNN heads qualify too with two request blocks (B > 32), their
        // hidden halves on the matrix cores, and a workgroup per rank column
        const int hd = Wrg != nullptr ? 2 : (Wg != nullptr ? 1 : 0);
        bool res_ok = mfma;
        if (hd == 1) res_ok = res_ok && B > 32 && gamma <= kResMaxGamma && hidden_mfma_ok(H, r, H + r, 0, h, Wg);
        if (hd == 2)
            res_ok = res_ok && B > 32 && gamma <= kResMaxGamma && hidden_mfma_ok(H, r, 2 * r + H, 2 * r, h, Wrg) &&
                     (uintptr_t)Wrc % 16 == 0;
        ResidentPlan rp = res_ok ? resident_plan(B, V, hd) : ResidentPlan{};
        if (hd != 0 && rp.nwg < kMfmaRank) rp.nwg = 0;
        // (stored logits or bias go to the general kernel: any store in the
        // resident kernel's tile loop makes its loads wait for one another)
        if (rp.nwg > 0 && lo == nullptr && bo == nullptr && (uintptr_t)U % 16 == 0 &&
            (G == nullptr || ((uintptr_t)G % 16 == 0 && B * gamma * V * 4 < ((int64_t)1 << 31)))) {
            char* p = static_cast<char*>(ws);
            uint32_t* header = reinterpret_cast<uint32_t*>(p);
            p += kResHeader;
            uint64_t* hword = reinterpret_cast<uint64_t*>(p);
            p += ((size_t)(8 * B * gamma) + 255) / 256 * 256;
            uint64_t* pub = reinterpret_cast<uint64_t*>(p);
            uint64_t* win = pub + (size_t)gamma * kResMaxWGs * kResMaxReq;
            float* hid = nullptr;
            uint64_t* ebw = nullptr;
            if (hd != 0) {
                char* q = static_cast<char*>(ws) + resident_workspace(B, gamma);
                hid = reinterpret_cast<float*>(q);
                ebw = reinterpret_cast<uint64_t*>(q + ((size_t)(4 * hd * kHidMaxSplits * B * gamma * kMfmaRank) + 255) /
                                                          256 * 256);
                const int64_t M = B * gamma;
                const int ks = hidden_splits(H, hd);
                const dim3 grid((uint32_t)(r / 32), (uint32_t)((M + 31) / 32), (uint32_t)(hd * ks));
                hipLaunchKernelGGL(hidden_mfma<kHidKU>, grid, dim3(64 * kHidWaves), 0, stream, M, H, r,
                                   hd == 2 ? 2 * r + H : H + r, hd == 2 ? 2 * r : (int64_t)0,
                                   static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(hd == 2 ? Wrg : Wg),
                                   static_cast<const bf16_t*>(Wrc), hid, hid + ks * M * r, ks, 1);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            int lim = wait_limit(kChainSpinLimit);
            int hks = hidden_splits(H, hd);
            const T* ht = static_cast<const T*>(h);
            const bf16_t* Wh = static_cast<const bf16_t*>(hd == 2 ? Wrg : Wg);
            const bf16_t* Wh2 = static_cast<const bf16_t*>(Wrc);
            int g = (int)gamma, tpw = rp.tiles_per_wg;
            int64_t Bb = B, Vv = V, Hh = H;
            void* args[] = {&Bb, &g,     &Vv,    &tpw,    &Ut,   &W1t,      &W2t,   &ht,  &wt,  &Hh,     &b_conf, &x0,
                            &G,  &force, &tokens, &conf, &survival, &hword, &pub, &win, &header, &lim, &Wh, &Wh2,
                            &hid, &hks, &ebw};
            const void* fn;
            if (hd == 1)
                fn = G ? reinterpret_cast<const void*>(&sample_batch_resident<2, true, 1>)
                       : reinterpret_cast<const void*>(&sample_batch_resident<2, false, 1>);
            else if (hd == 2)
                fn = G ? reinterpret_cast<const void*>(&sample_batch_resident<2, true, 2>)
                       : reinterpret_cast<const void*>(&sample_batch_resident<2, false, 2>);
            else
                fn = G ? (B <= 32 ? reinterpret_cast<const void*>(&sample_batch_resident<1, true, 0>)
                                  : reinterpret_cast<const void*>(&sample_batch_resident<2, true, 0>))
                       : (B <= 32 ? reinterpret_cast<const void*>(&sample_batch_resident<1, false, 0>)
                                  : reinterpret_cast<const void*>(&sample_batch_resident<2, false, 0>));
            // a plain launch: one workgroup per CU at most, all resident together;
            // the bounded spins turn any other outcome into an error, not a hang
            return hipLaunchKernel(fn, dim3(rp.nwg), dim3(kResThreads), args, 0, stream);
        }
    }
    const int ncopy = mfma ? kKeyCopies : 1;
    Buffers s = carve(ws, B, gamma, ncopy);

    hipLaunchKernelGGL((sample_init<T>), dim3((uint32_t)(B * gamma)), dim3(kThreads), 0, stream, B, gamma, H,
                       static_cast<const T*>(h), wt, s.keys, ncopy, s.hdot);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // scratch of the gated and RNN heads after the hidden dots.  Gated: the
    // gate's hidden halves [B][gamma][r], then the gated embeddings of the
    // current step [B][r].  RNN: the two hidden halves [2][B][gamma][r], then
    // two state buffers [2][B][r] (step k writes buffer k % 2).
    const T* Wgt = static_cast<const T*>(Wg);
    const T* Wrgt = static_cast<const T*>(Wrg);
    const T* Wrct = static_cast<const T*>(Wrc);
    const bool rnn = Wrg != nullptr;
    float* gate_ws = (Wg || rnn) ? s.hdot + ((B * gamma + 63) / 64) * 64 : nullptr;
    const int64_t gate_words = (rnn ? 2 * gamma + 2 : gamma + 1) * r;  // per request
    // the hidden halves: a bf16 contraction [B gamma, H] x [H, r] on the
    // matrix cores where the shapes allow, else one wave per dot
    bool hmfma = false;
    if constexpr (std::is_same_v<T, bf16_t>) {
        if (rnn)
            hmfma = hidden_mfma_ok(H, r, 2 * r + H, 2 * r, h, Wrg) && (uintptr_t)Wrc % 16 == 0;
        else if (Wg)
            hmfma = hidden_mfma_ok(H, r, H + r, 0, h, Wg);
        if (hmfma) {
            const int64_t M = B * gamma;
            const dim3 grid((uint32_t)(r / 32), (uint32_t)((M + 31) / 32), rnn ? 2u : 1u);
            hipLaunchKernelGGL(hidden_mfma<kHidKU>, grid, dim3(64 * kHidWaves), 0, stream, M, H, r,
                               rnn ? 2 * r + H : H + r, rnn ? 2 * r : (int64_t)0, static_cast<const bf16_t*>(h),
                               static_cast<const bf16_t*>(rnn ? Wrg : Wg), static_cast<const bf16_t*>(Wrc), gate_ws,
                               gate_ws + B * gamma * r, 1, 0);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if (rnn && !hmfma) {
        const dim3 grid((uint32_t)(B * gamma), (uint32_t)((r + kGateRows - 1) / kGateRows));
        hipLaunchKernelGGL((rnn_hidden<T>), grid, dim3(kThreads), 0, stream, H, r, static_cast<const T*>(h), Wrgt,
                           Wrct, gate_ws, gate_ws + B * gamma * r);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (Wg && !hmfma) {
        const dim3 grid((uint32_t)(B * gamma), (uint32_t)((r + kGateRows - 1) / kGateRows));
        hipLaunchKernelGGL((gate_hidden<T>), grid, dim3(kThreads), 0, stream, H, r, static_cast<const T*>(h), Wgt,
                           gate_ws);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    // bf16 gate and state steps with every lane's rank elements in one 16-byte piece
    bool fast_gate = false, fast_rnn = false;
    if constexpr (std::is_same_v<T, bf16_t>) {
        const bool rows16 = r % 8 == 0 && H % 8 == 0 && (uintptr_t)W1 % 16 == 0;
        fast_gate = Wg && rows16 && r <= 512 && (uintptr_t)Wg % 16 == 0;
        fast_rnn = rnn && rows16 && r <= 256 && (uintptr_t)Wrg % 16 == 0 && (uintptr_t)Wrc % 16 == 0 &&
                   (uintptr_t)ws % 16 == 0;
    }

    // lanes per W2 row: 16-byte chunks per row when rows are 16-byte aligned
    const int64_t row_bytes = r * (int64_t)sizeof(T);
    int lpr = 0;
    if (row_bytes % 16 == 0 && row_bytes / 16 <= 64 && (((uintptr_t)W2) % 16 == 0)) {
        const int64_t q = row_bytes / 16;
        if ((q & (q - 1)) == 0) lpr = (int)q;
    }
    for (int k = 0; k < gamma; ++k) {
        const float* eg = nullptr;
        if (Wg) {
            const dim3 grid((uint32_t)B, (uint32_t)((r + kGateRows - 1) / kGateRows));
            if (fast_gate)
                hipLaunchKernelGGL(gate_step_bf16, grid, dim3(kThreads), 0, stream, B, gamma, k, V, H, r,
                                   reinterpret_cast<const bf16_t*>(W1t), reinterpret_cast<const bf16_t*>(Wgt), x0,
                                   force, s.keys, ncopy, gate_ws, gate_ws + B * gamma * r);
            else
                hipLaunchKernelGGL((gate_step<T>), grid, dim3(kThreads), 0, stream, B, gamma, k, V, H, r, W1t, Wgt,
                                   x0, force, s.keys, ncopy, gate_ws, gate_ws + B * gamma * r);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            eg = gate_ws + B * gamma * r;
        }
        if (rnn) {
            float* st = gate_ws + 2 * B * gamma * r;
            const dim3 grid((uint32_t)B, (uint32_t)((r + kGateRows - 1) / kGateRows));
            if (fast_rnn)
                hipLaunchKernelGGL(rnn_step_bf16, grid, dim3(kThreads), 0, stream, B, gamma, k, V, H, r,
                                   reinterpret_cast<const bf16_t*>(W1t), reinterpret_cast<const bf16_t*>(Wrgt),
                                   reinterpret_cast<const bf16_t*>(Wrct), x0, force, s.keys, ncopy, gate_ws,
                                   gate_ws + B * gamma * r, st + ((k + 1) % 2) * B * r, st + (k % 2) * B * r);
            else
                hipLaunchKernelGGL((rnn_step<T>), grid, dim3(kThreads), sizeof(float) * 2 * r, stream, B, gamma, k, V,
                                   H, r, W1t, Wrgt, Wrct, x0, force, s.keys, ncopy, gate_ws, gate_ws + B * gamma * r,
                                   st + ((k + 1) % 2) * B * r, st + (k % 2) * B * r);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            eg = st + (k % 2) * B * r;
        }
        if constexpr (std::is_same_v<T, bf16_t>) {
            if (mfma) {
                const dim3 grid((uint32_t)((V + kMfmaRows - 1) / kMfmaRows), (uint32_t)((B + 63) / 64));
                // coalesced tiles need 16-byte aligned U and G rows
                const bool stage = V % 8 == 0 && (uintptr_t)U % 16 == 0 && (G == nullptr || (uintptr_t)G % 16 == 0);
#define DSPARK_MFMA(NT, ST, EG)                                                                                   \
    hipLaunchKernelGGL((sample_step_mfma<NT, ST, EG>), grid, dim3(256), 0, stream, B, gamma, k, V, Ut, W1t, W2t, G, \
                       x0, force, s.keys, lo, bo, eg)
                if (eg) {
                    if (B <= 32) {
                        if (stage) DSPARK_MFMA(1, true, true); else DSPARK_MFMA(1, false, true);
                    } else {
                        if (stage) DSPARK_MFMA(2, true, true); else DSPARK_MFMA(2, false, true);
                    }
                } else if (B <= 32) {
                    if (stage) DSPARK_MFMA(1, true, false); else DSPARK_MFMA(1, false, false);
                } else {
                    if (stage) DSPARK_MFMA(2, true, false); else DSPARK_MFMA(2, false, false);
                }
#undef DSPARK_MFMA
                err = hipGetLastError();
                if (err != hipSuccess) return err;
                continue;
            }
        }
        if (B == 1)
            err = launch_steps<T, 1>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, eg, stream);
        else if (B == 2)
            err = launch_steps<T, 2>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, eg, stream);
        else if (B <= 4)
            err = launch_steps<T, 4>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, eg, stream);
        else
            err = launch_steps<T, 8>(lpr, B, gamma, k, V, r, Ut, W1t, W2t, G, x0, force, s.keys, lo, bo, eg, stream);
        if (err != hipSuccess) return err;
    }
    const int fwaves = gamma < kFinishMaxGamma ? (int)gamma : kFinishMaxGamma;
    hipLaunchKernelGGL((sample_finish<T>), dim3((uint32_t)B), dim3(64 * fwaves), 0, stream, B, gamma, V, H, r, W1t, wt,
                       b_conf, x0, force, s.keys, ncopy, s.hdot, tokens, conf, survival);
    if (Wg || rnn) {  // the gate words go back to zero for the next call
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(clear_words, dim3((uint32_t)((B * gate_words + kThreads - 1) / kThreads)), dim3(kThreads),
                           0, stream, gate_ws, B * gate_words);
    }
    return hipGetLastError();
}

}  // namespace

size_t head_sample_workspace(int64_t B, int64_t gamma, int64_t, int64_t r, int dtype) {
    const int64_t ncopy = (dtype == kBF16 && r == kMfmaRank && B >= kMfmaMinBatch) ? kKeyCopies : 1;
    size_t steps = kWsHeader + ((size_t)(8 * kKeyStride * ncopy * B * gamma) + 255) / 256 * 256 +
                   ((size_t)(4 * B * gamma) + 255) / 256 * 256;
    if (dtype == kBF16 && r == kMfmaRank && B >= kMfmaMinBatch && B <= kResMaxReq) {
        const size_t res = resident_workspace(B, gamma);
        if (res > steps) steps = res;
    }
    if (B == 1 && r == kChainRank) {
        const size_t chain = chain_workspace(gamma);
        if (chain > steps) steps = chain;
    }
    return steps;
}

// the per-step path's keys (kKeyCopies copies on the matrix-core path, else
// one) and hidden dots, then a gated or RNN head's words
size_t headed_workspace(int64_t B, int64_t gamma, int64_t r, int dtype, int64_t words_per_request) {
    const int64_t ncopy = (dtype == kBF16 && r == kMfmaRank && B >= kMfmaMinBatch) ? kKeyCopies : 1;
    return kWsHeader + ((size_t)(8 * kKeyStride * ncopy * B * gamma) + 255) / 256 * 256 +
           ((size_t)(4 * B * gamma) + 255) / 256 * 256 + ((size_t)(4 * B * words_per_request) + 255) / 256 * 256;
}

size_t head_sample_gated_workspace(int64_t B, int64_t gamma, int64_t r, int dtype) {
    size_t w = headed_workspace(B, gamma, r, dtype, (gamma + 1) * r);
    if (dtype == kBF16 && r == kMfmaRank && B > 32 && B <= kResMaxReq && gamma <= kResMaxGamma) {
        const size_t res = resident_head_workspace(B, gamma, 1);
        if (res > w) w = res;
    }
    return w;
}

size_t head_sample_rnn_workspace(int64_t B, int64_t gamma, int64_t r, int dtype) {
    size_t w = headed_workspace(B, gamma, r, dtype, (2 * gamma + 2) * r);
    if (dtype == kBF16 && r == kMfmaRank && B > 32 && B <= kResMaxReq && gamma <= kResMaxGamma) {
        const size_t res = resident_head_workspace(B, gamma, 2);
        if (res > w) w = res;
    }
    return w;
}

hipError_t w2_bound_launch(int64_t V, const void* W2, uint32_t* out, hipStream_t stream) {
    const bf16_t* W2t = static_cast<const bf16_t*>(W2);
    hipLaunchKernelGGL(w2_bound_init, dim3(1), dim3(kChainThreads), 0, stream, V, W2t, out);
    const int cus = device_cus() > 0 ? device_cus() : 1;
    const int64_t need = (V + 4 * kSampleRows - 1) / (4 * kSampleRows);
    const int grid = (int)(need < 4 * (int64_t)cus ? need : 4 * (int64_t)cus);
    hipLaunchKernelGGL(w2_bound_max, dim3(grid > 0 ? grid : 1), dim3(kChainThreads), 0, stream, V, W2t, out);
    hipLaunchKernelGGL(w2_bound_tag, dim3(1), dim3(64), 0, stream, out);
    return hipGetLastError();
}

hipError_t head_sample_launch(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int dtype, const void* U,
                              const void* h, const void* W1, const void* W2, const void* w_conf, float b_conf,
                              const int32_t* x0, const float* gumbel, const int32_t* force, int32_t* tokens,
                              float* conf, float* survival, float* logits_out, float* bias_out, void* ws,
                              hipStream_t stream, const void* Wg, const void* Wrg, const void* Wrc,
                              const uint32_t* w2_bound) {
    if (Wg == nullptr && Wrg == nullptr && chain_eligible(B, r, dtype, W1, W2)) {
        const ChainPlan p = chain_plan(V, H);
        if (p.nwg > 0)
            return launch_chain(p, gamma, V, H, U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, tokens, conf,
                                survival, logits_out, bias_out, ws, stream, w2_bound);
    }
    if (dtype == kBF16)
        return launch_typed<bf16_t>(B, gamma, V, H, r, U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, tokens,
                                    conf, survival, logits_out, bias_out, ws, stream, Wg, Wrg, Wrc);
    return launch_typed<float>(B, gamma, V, H, r, U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, tokens, conf,
                               survival, logits_out, bias_out, ws, stream, Wg, Wrg, Wrc);
}

}  // namespace dspark
