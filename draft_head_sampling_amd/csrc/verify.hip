// Rejection-sampling verification of one draft block per request
// ("基于 DSpark 的投机解码训练框架原理与实现", wangjunjian.com: section 8.2,
// the verification rule; section 2.1, the bonus token the target adds after
// an accepted prefix).
//
// Request b drafted n = n_draft[b] tokens x_1..x_n.  Position k keeps x_k iff
// u_k * p_d(x_k) < p_t(x_k), i.e. u_k < min(1, p_t(x_k) / p_d(x_k)), with
// p_d = softmax(d[b,k,:]) and p_t = softmax(t[b,k,:]).  The first rejection
// ends the block and the next token is drawn from the residual
// max(0, p_t - p_d) at that position; when every drafted token is kept the
// next token is the bonus draw from p_t at position n + 1.  Both draws are
// Gumbel-max with the request's noise row G[b,:]:
//   residual  argmax over v with p_t(v) > p_d(v) of ln(p_t(v) - p_d(v)) + G_v
//   bonus     argmax of t[b,n+1,v] + G_v
// (an empty residual falls back to the p_t draw at the same position).
//
// Two launches on the caller's stream:
//   verify_stats   four workgroups per drafted (request, position) row pair:
//                  each a quarter of both rows' online (max, sum of exp),
//                  binary32
//   verify_sample  (vocabulary chunk, request) workgroups: the accept walk
//                  (one lane per position), then the chunk's part of the draw
//                  as packed argmax keys (score high, complemented id low)
//                  in the workgroup's own slot; the last workgroup of a
//                  request to arrive merges the slots, decodes the token and
//                  clears the request's workspace words for the next call
// Only the sampled position's rows are read twice; every other row once.
#include "internal.h"

namespace dspark {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStatThreads = 512;
constexpr int kStatUnroll = 4;  // 16-byte vectors of each row in flight per thread
constexpr int kSampleThreads = 256;
constexpr int kSampleVecs = 4;  // vectors per thread per sampling workgroup

// Workspace: per (request, position, row split) the two rows' partial
// (max, sum of exp) as four binary32 words; per (request, vocabulary chunk)
// a slot of two argmax keys (residual, p_t); per request an arrival counter
// of the sampling workgroups; all after the common 256-byte header, whose
// word 1 is the give-up status.
constexpr int kSplit = 4;  // workgroups per (request, position) row pair
constexpr size_t kStatWords = 4;
constexpr uint64_t kNoKey = 1;  // a written slot word without a candidate (below every real key)
constexpr int kSpinLimit = 1 << 22;

// vocabulary chunks of the sampling launch, at most (the unvectorised span)
int64_t max_chunks(int64_t V) { return (V + kSampleThreads * kSampleVecs - 1) / (kSampleThreads * kSampleVecs); }
size_t stats_bytes(int64_t B, int64_t gamma) {
    return ((size_t)(B * gamma) * kSplit * kStatWords * 4 + 255) / 256 * 256;
}
size_t slots_bytes(int64_t B, int64_t V) { return ((size_t)B * max_chunks(V) * 16 + 255) / 256 * 256; }
size_t count_bytes(int64_t B) { return ((size_t)B * 4 + 255) / 256 * 256; }

template <typename T>
struct Vec;
template <>
struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const uint4& r, float (&x)[4]) {
        x[0] = __uint_as_float(r.x), x[1] = __uint_as_float(r.y), x[2] = __uint_as_float(r.z),
        x[3] = __uint_as_float(r.w);
    }
};
template <>
struct Vec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void unpack(const uint4& r, float (&x)[8]) {
        x[0] = widen_lo(r.x), x[1] = widen_hi(r.x), x[2] = widen_lo(r.y), x[3] = widen_hi(r.y);
        x[4] = widen_lo(r.z), x[5] = widen_hi(r.z), x[6] = widen_lo(r.w), x[7] = widen_hi(r.w);
    }
};

// Running (max, sum of exp(x - max)), folded in groups of n values.
template <int N>
__device__ __forceinline__ void fold(float& m, float& s, const float (&x)[N]) {
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
    const float mn = fmaxf(m, bm);
    const float mnl = mn * kLog2e;
    float acc = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -mnl));
#pragma unroll
    for (int i = 0; i < N; ++i) acc += exp_shifted(x[i], mnl);
    s = mn == -INFINITY ? 0.f : acc;  // nothing but -inf so far: an empty sum
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
__device__ void block_merge2(float& m1, float& s1, float& m2, float& s2, float* lds) {
    for (int o = 32; o > 0; o >>= 1) {
        merge(m1, s1, __shfl_xor(m1, o), __shfl_xor(s1, o));
        merge(m2, s2, __shfl_xor(m2, o), __shfl_xor(s2, o));
    }
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) lds[4 * w] = m1, lds[4 * w + 1] = s1, lds[4 * w + 2] = m2, lds[4 * w + 3] = s2;
    __syncthreads();
    m1 = lds[0], s1 = lds[1], m2 = lds[2], s2 = lds[3];
    for (int i = 1; i < NT / 64; ++i) merge(m1, s1, lds[4 * i], lds[4 * i + 1]), merge(m2, s2, lds[4 * i + 2], lds[4 * i + 3]);
}

__device__ __forceinline__ int32_t clamp_n(const int32_t* n_draft, int64_t b, int64_t gamma) {
    int64_t n = n_draft ? n_draft[b] : gamma;
    return (int32_t)(n < 0 ? 0 : n > gamma ? gamma : n);
}

// One workgroup per (request, drafted position, row split): the split's
// partial (max, sum) of the draft row and of the target row.
// VEC: rows start on 16-byte boundaries and V is a whole number of vectors.
template <typename T, bool VEC>
__global__ __launch_bounds__(kStatThreads) void verify_stats(int64_t gamma, int64_t V, const T* __restrict__ d,
                                                             const T* __restrict__ t,
                                                             const int32_t* __restrict__ n_draft, float* stats) {
    __shared__ float lds[4 * kStatThreads / 64];
    const int64_t row = blockIdx.x / kSplit;
    const int sp = blockIdx.x % kSplit;
    const int64_t b = row / gamma, k = row % gamma;
    const int tid = threadIdx.x;
    if (k >= clamp_n(n_draft, b, gamma)) return;  // not drafted: nothing to verify
    const T* dr = d + (b * gamma + k) * V;
    const T* tr = t + (b * (gamma + 1) + k) * V;
    float md = -INFINITY, sd = 0.f, mt = -INFINITY, st = 0.f;
    if (VEC) {
        constexpr int E = Vec<T>::N;
        const int64_t nvec = V / E;
        const int64_t per = (nvec + kSplit - 1) / kSplit;
        const int64_t lo = sp * per, hi = lo + per < nvec ? lo + per : nvec;
        const uint4* dv = reinterpret_cast<const uint4*>(dr);
        const uint4* tv = reinterpret_cast<const uint4*>(tr);
        for (int64_t base = lo; base < hi; base += (int64_t)kStatThreads * kStatUnroll) {
            // unconditional loads from clamped indices, masked afterwards: the
            // compiler then waits for each vector as it is folded
            uint4 rd[kStatUnroll], rt[kStatUnroll];
            bool in[kStatUnroll];
#pragma unroll
            for (int j = 0; j < kStatUnroll; ++j) {
                const int64_t i = base + tid + (int64_t)j * kStatThreads;
                in[j] = i < hi;
                rd[j] = dv[in[j] ? i : lo];
                rt[j] = tv[in[j] ? i : lo];
            }
#pragma unroll
            for (int j = 0; j < kStatUnroll; ++j) {
                float xd[E], xt[E];
                Vec<T>::unpack(rd[j], xd);
                Vec<T>::unpack(rt[j], xt);
                float md2 = md, sd2 = sd, mt2 = mt, st2 = st;
                fold<E>(md2, sd2, xd);
                fold<E>(mt2, st2, xt);
                md = in[j] ? md2 : md, sd = in[j] ? sd2 : sd;
                mt = in[j] ? mt2 : mt, st = in[j] ? st2 : st;
            }
        }
    } else {
        const int64_t per = (V + kSplit - 1) / kSplit;
        const int64_t lo = sp * per, hi = lo + per < V ? lo + per : V;
        for (int64_t v = lo + tid; v < hi; v += kStatThreads) {
            float xd[1] = {load_elem(dr, v)}, xt[1] = {load_elem(tr, v)};
            fold<1>(md, sd, xd);
            fold<1>(mt, st, xt);
        }
    }
    block_merge2<kStatThreads>(md, sd, mt, st, lds);
    if (tid == 0) {
        float* s = stats + ((b * gamma + k) * kSplit + sp) * kStatWords;
        s[0] = md, s[1] = sd, s[2] = mt, s[3] = st;
    }
}

// (vocabulary chunk, request) workgroups.  Wave 0 first redoes the request's
// accept walk, one lane per drafted position: it merges the splits' partials
// into the two log2-normalisers, takes p_d and p_t of the drafted token and
// keeps the token while u * p_d < p_t; the first lane that fails is the
// rejected position.  (Chunk 0 also writes n_accepted and accept_prob.)
// Then the chunk's part of the draw: the packed argmax keys of the residual
// and of the p_t draw, stored in the workgroup's own slot (a written word is
// never zero).  A relaxed arrival counter elects the request's last
// workgroup, which waits for every slot, takes the maximum, decodes the
// token and clears the request's workspace words for the next call.  No
// exchange needs a fence.
template <typename T, bool VEC>
__global__ __launch_bounds__(kSampleThreads) void verify_sample(
    int64_t gamma, int64_t V, const T* __restrict__ d, const T* __restrict__ t, const int32_t* __restrict__ x,
    const int32_t* __restrict__ n_draft, const float* __restrict__ u, const float* __restrict__ G, float* stats,
    uint64_t* slots, uint32_t* counters, int32_t* __restrict__ n_accepted, float* __restrict__ accept_prob,
    int32_t* __restrict__ next_token, uint32_t* header, int spin_limit) {
    static_assert(kSampleThreads >= 64, "wave 0 walks the positions");
    __shared__ uint64_t red[2][kSampleThreads / 64];
    __shared__ int s_pos, s_res;
    __shared__ float s_cd, s_ct;
    __shared__ int s_last;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t n = clamp_n(n_draft, b, gamma);
    constexpr int E = Vec<T>::N;
    const float* g = G + b * V;
    // the Gumbel row does not depend on the walk: its loads go out first
    float4 rg[kSampleVecs][E / 4];
    if (VEC) {
        const int64_t nvec = V / E;
        const int64_t v0 = (int64_t)blockIdx.x * kSampleThreads * kSampleVecs;
#pragma unroll
        for (int j = 0; j < kSampleVecs; ++j) {
            const int64_t i = v0 + tid + (int64_t)j * kSampleThreads;
            const int64_t ic = i < nvec ? i : 0;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) rg[j][q] = reinterpret_cast<const float4*>(g)[ic * (E / 4) + q];
        }
    }
    if (wave == 0) {
        int pos = n, res = 0;
        float cdp = 0.f, ctp = 0.f;
        for (int64_t k0 = 0; k0 < n; k0 += 64) {  // 64 positions per round (gamma <= 4096)
            const int64_t k = k0 + lane;
            const bool act = k < n;
            float cd = 0.f, ct = 0.f, pd = 0.f, pt = 0.f;
            bool keep = false, valid = false;
            if (act) {
                float md = -INFINITY, sd = 0.f, mt = -INFINITY, st = 0.f;
                const float* s = stats + (b * gamma + k) * kSplit * kStatWords;
                for (int q = 0; q < kSplit; ++q) {
                    merge(md, sd, s[q * kStatWords + 0], s[q * kStatWords + 1]);
                    merge(mt, st, s[q * kStatWords + 2], s[q * kStatWords + 3]);
                }
                cd = md * kLog2e + __builtin_amdgcn_logf(sd);
                ct = mt * kLog2e + __builtin_amdgcn_logf(st);
                const int32_t xk = x[b * gamma + k];
                valid = xk >= 0 && xk < V;
                pd = valid ? exp_shifted(load_elem(d + (b * gamma + k) * V, xk), cd) : 0.f;
                pt = valid ? exp_shifted(load_elem(t + (b * (gamma + 1) + k) * V, xk), ct) : 0.f;
                keep = valid && u[b * gamma + k] * pd < pt;
                if (blockIdx.x == 0 && accept_prob)
                    accept_prob[b * gamma + k] = !valid ? 0.f : pd > 0.f ? fminf(1.f, pt / pd) : (pt > 0.f ? 1.f : 0.f);
            }
            const uint64_t fails = __ballot(act && !keep);
            if (pos == n && fails) {
                const int j = __builtin_ctzll(fails);
                pos = (int)(k0 + j), res = 1;
                cdp = __shfl(cd, j), ctp = __shfl(ct, j);
            }
        }
        if (lane == 0) {
            s_pos = pos, s_res = res, s_cd = cdp, s_ct = ctp;
            if (blockIdx.x == 0) n_accepted[b] = pos;
        }
        if (blockIdx.x == 0 && accept_prob)
            for (int64_t k = n + lane; k < gamma; k += 64) accept_prob[b * gamma + k] = __builtin_nanf("");
    }
    __syncthreads();
    const int64_t pos = s_pos;
    const bool res = s_res != 0;
    const float cd = s_cd, ct = s_ct;
    const T* tr = t + (b * (gamma + 1) + pos) * V;
    const T* dr = d + (b * gamma + (res ? pos : 0)) * V;  // read only for a residual draw
    uint64_t kr = 0, kt = 0;  // residual and p_t keys
    auto consider = [&](float xt, float xd, float gv, int64_t v) {
        kt = umax64(kt, argmax_key(xt + gv, (uint32_t)v));
        if (res) {
            const float r = exp_shifted(xt, ct) - exp_shifted(xd, cd);
            const float sc = __builtin_fmaf(__builtin_amdgcn_logf(r), kLn2, gv);
            kr = r > 0.f ? umax64(kr, argmax_key(sc, (uint32_t)v)) : kr;
        }
    };
    if (VEC) {
        const int64_t nvec = V / E;
        const int64_t v0 = (int64_t)blockIdx.x * kSampleThreads * kSampleVecs;
        uint4 rt[kSampleVecs], rd[kSampleVecs];
        bool in[kSampleVecs];
#pragma unroll
        for (int j = 0; j < kSampleVecs; ++j) {
            const int64_t i = v0 + tid + (int64_t)j * kSampleThreads;
            in[j] = i < nvec;
            const int64_t ic = in[j] ? i : 0;
            rt[j] = reinterpret_cast<const uint4*>(tr)[ic];
            rd[j] = res ? reinterpret_cast<const uint4*>(dr)[ic] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kSampleVecs; ++j) {
            if (!in[j]) continue;
            float xt[E], xd[E];
            Vec<T>::unpack(rt[j], xt);
            Vec<T>::unpack(rd[j], xd);
            const int64_t v = (v0 + tid + (int64_t)j * kSampleThreads) * E;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                consider(xt[4 * q + 0], xd[4 * q + 0], rg[j][q].x, v + 4 * q + 0);
                consider(xt[4 * q + 1], xd[4 * q + 1], rg[j][q].y, v + 4 * q + 1);
                consider(xt[4 * q + 2], xd[4 * q + 2], rg[j][q].z, v + 4 * q + 2);
                consider(xt[4 * q + 3], xd[4 * q + 3], rg[j][q].w, v + 4 * q + 3);
            }
        }
    } else {
        const int64_t span = (int64_t)kSampleThreads * kSampleVecs;
        const int64_t v0 = (int64_t)blockIdx.x * span;
        const int64_t v1 = v0 + span < V ? v0 + span : V;
        for (int64_t v = v0 + tid; v < v1; v += kSampleThreads)
            consider(load_elem(tr, v), res ? load_elem(dr, v) : 0.f, g[v], v);
    }
    for (int o = 32; o > 0; o >>= 1) {
        kr = umax64(kr, (uint64_t)__shfl_xor((unsigned long long)kr, o));
        kt = umax64(kt, (uint64_t)__shfl_xor((unsigned long long)kt, o));
    }
    if (lane == 0) red[0][wave] = kr, red[1][wave] = kt;
    __syncthreads();
    const int nch = gridDim.x;
    uint64_t* slot = slots + ((int64_t)b * nch + blockIdx.x) * 2;
    if (tid == 0) {
        for (int w = 1; w < kSampleThreads / 64; ++w) kr = umax64(kr, red[0][w]), kt = umax64(kt, red[1][w]);
        __hip_atomic_store(slot, kr ? kr : kNoKey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, kt ? kt : kNoKey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t old = __hip_atomic_fetch_add(counters + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)nch - 1;
    }
    __syncthreads();
    if (s_last && wave == 0) {
        // every other workgroup has arrived; wait until its slot words are seen
        uint64_t mr = 0, mt = 0;
        bool ok = false;
        const uint64_t* req = slots + (int64_t)b * nch * 2;
        for (int spin = 0; spin < spin_limit; ++spin) {
            bool all = true;
            mr = 0, mt = 0;
            for (int c = lane; c < nch; c += 64) {
                const uint64_t a0 = __hip_atomic_load(req + 2 * c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t a1 = __hip_atomic_load(req + 2 * c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                all = all && a0 != 0 && a1 != 0;
                mr = umax64(mr, a0), mt = umax64(mt, a1);
            }
            ok = __all(all);
            if (ok) break;
            __builtin_amdgcn_s_sleep(1);
        }
        for (int o = 32; o > 0; o >>= 1) {
            mr = umax64(mr, (uint64_t)__shfl_xor((unsigned long long)mr, o));
            mt = umax64(mt, (uint64_t)__shfl_xor((unsigned long long)mt, o));
        }
        if (lane == 0) {
            const uint64_t k = res && mr > kNoKey ? mr : mt;
            next_token[b] = ok && k > kNoKey ? key_token(k) : -1;
            if (!ok) mark_gave_up(header);
            __hip_atomic_store(counters + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int c = lane; c < 2 * nch; c += 64)
            __hip_atomic_store(slots + (int64_t)b * nch * 2 + c, (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        for (int64_t i = lane; i < gamma * kSplit * (int64_t)kStatWords; i += 64)
            stats[b * gamma * kSplit * kStatWords + i] = 0.f;
    }
}

template <typename T>
hipError_t launch_typed(int64_t B, int64_t gamma, int64_t V, const void* d, const void* t, const int32_t* x,
                        const int32_t* n_draft, const float* u, const float* G, int32_t* n_accepted,
                        int32_t* next_token, float* accept_prob, void* ws, hipStream_t stream) {
    constexpr int E = Vec<T>::N;
    const T* dp = static_cast<const T*>(d);
    const T* tp = static_cast<const T*>(t);
    const bool vec = V % E == 0 && (uintptr_t)d % 16 == 0 && (uintptr_t)t % 16 == 0 && (uintptr_t)G % 16 == 0;
    uint32_t* header = static_cast<uint32_t*>(ws);  // word 1: a lost slot (bounded wait ran out) -> token -1
    char* w = static_cast<char*>(ws) + kWsHeader;
    float* stats = reinterpret_cast<float*>(w);
    uint64_t* slots = reinterpret_cast<uint64_t*>(w + stats_bytes(B, gamma));
    uint32_t* counters = reinterpret_cast<uint32_t*>(w + stats_bytes(B, gamma) + slots_bytes(B, V));
    const int lim = wait_limit(kSpinLimit);
    if (gamma > 0) {
        const dim3 grid((uint32_t)(B * gamma * kSplit));
        if (vec)
            hipLaunchKernelGGL((verify_stats<T, true>), grid, dim3(kStatThreads), 0, stream, gamma, V, dp, tp,
                               n_draft, stats);
        else
            hipLaunchKernelGGL((verify_stats<T, false>), grid, dim3(kStatThreads), 0, stream, gamma, V, dp, tp,
                               n_draft, stats);
    }
    const int64_t span = vec ? (int64_t)kSampleThreads * kSampleVecs * E : (int64_t)kSampleThreads * kSampleVecs;
    const dim3 sgrid((uint32_t)((V + span - 1) / span), (uint32_t)B);
    if (vec)
        hipLaunchKernelGGL((verify_sample<T, true>), sgrid, dim3(kSampleThreads), 0, stream, gamma, V, dp, tp, x,
                           n_draft, u, G, stats, slots, counters, n_accepted, accept_prob, next_token, header, lim);
    else
        hipLaunchKernelGGL((verify_sample<T, false>), sgrid, dim3(kSampleThreads), 0, stream, gamma, V, dp, tp, x,
                           n_draft, u, G, stats, slots, counters, n_accepted, accept_prob, next_token, header, lim);
    return hipGetLastError();
}

}  // namespace

size_t verify_workspace(int64_t B, int64_t gamma, int64_t V) {
    return kWsHeader + stats_bytes(B, gamma) + slots_bytes(B, V) + count_bytes(B);
}

hipError_t verify_launch(int64_t B, int64_t gamma, int64_t V, int dtype, const void* d, const void* t,
                         const int32_t* x, const int32_t* n_draft, const float* u, const float* G,
                         int32_t* n_accepted, int32_t* next_token, float* accept_prob, void* ws, hipStream_t stream) {
    if (dtype == kBF16)
        return launch_typed<bf16_t>(B, gamma, V, d, t, x, n_draft, u, G, n_accepted, next_token, accept_prob, ws,
                                    stream);
    return launch_typed<float>(B, gamma, V, d, t, x, n_draft, u, G, n_accepted, next_token, accept_prob, ws, stream);
}

}  // namespace dspark
