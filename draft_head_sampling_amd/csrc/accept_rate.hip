// Analytic accept rate, paper eq. 8 ("基于 DSpark 的投机解码训练框架原理与实现",
// wangjunjian.com, section 3.3):
//     c*_n = 1 - 1/2 * || softmax(d_n) - softmax(t_n) ||_1
// an HBM-bound two-pass reduction over each row pair.
//
// Pass 1 keeps a running (max, sum of exp(x - max)) per thread for both rows,
// folding each loaded vector in with one rescale; the per-thread pairs are
// then merged.  Pass 2 accumulates |p - q| with the row statistics, the
// normaliser folded into the exponent: p = exp2(x log2 e - (m log2 e +
// log2 s)).  All sums are binary32, reduced in a fixed order, so results are
// bitwise reproducible.
//
// Cluster kernel (rows 16-byte aligned): a row pair is split over a cluster
// of C co-resident workgroups.  Each keeps its chunk of both rows in
// registers between the passes, so every logit crosses HBM once.  The
// clusters' (max, sum) statistics meet in slots tagged with the row's
// iteration number (a word is valid when its tag matches; two slot sets
// alternate between consecutive rows).  The partial L1 terms are tagged words
// as well; the last workgroup of a cluster to finish a row -- elected by one
// relaxed atomic add -- waits for all C tags, sums the terms in chunk order
// and writes the result.  No exchange needs a memory fence.  The grid never exceeds what fits on the
// GPU at once, and every wait is bounded; the last workgroup to leave clears
// the slots and counters for the next call.
//
// Row kernel (any alignment): one workgroup per row pair; pass 2 re-reads the
// rows.
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


// ---------------------------------------------------------------------------
// Cluster kernel
// ---------------------------------------------------------------------------
constexpr int kCThreads = 256;
constexpr int kCMaxVec = 10;     // 16-byte vectors per thread per row chunk
constexpr int kCMaxCluster = 16;
constexpr int kCSpinLimit = 1 << 22;
constexpr size_t kCHeader = kWsHeader;  // words 0 (exit counter), 1 (status), 2 (row counter), 3 (paths)

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& r, float (&x)[Vec<T>::N]);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& r, float (&x)[4]) {
    x[0] = __uint_as_float(r.x), x[1] = __uint_as_float(r.y), x[2] = __uint_as_float(r.z), x[3] = __uint_as_float(r.w);
}
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& r, float (&x)[8]) {
    x[0] = widen_lo(r.x), x[1] = widen_hi(r.x), x[2] = widen_lo(r.y), x[3] = widen_hi(r.y);
    x[4] = widen_lo(r.z), x[5] = widen_hi(r.z), x[6] = widen_lo(r.w), x[7] = widen_hi(r.w);
}

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) { return ((uint64_t)tag << 32) | __float_as_uint(v); }

template <typename T, int NV>
__global__ __launch_bounds__(kCThreads) void accept_rate_cluster(int64_t N, int64_t V, int C, int n_clusters,
                                                                 int64_t vpc, const T* __restrict__ d, int64_t ldd,
                                                                 const T* __restrict__ t, int64_t ldt,
                                                                 float* __restrict__ out, uint64_t* stats,
                                                                 uint64_t* parts, uint32_t* counters, uint64_t* nexts,
                                                                 uint32_t* header, int spin_limit) {
    static_assert(kCMaxCluster * 4 <= 64, "one wave polls all statistics words of a cluster");
    __shared__ float lds[2 * kCThreads / 64];
    __shared__ float rowstat[4];
    __shared__ int64_t next_row;
    __shared__ int last_flag;
    constexpr int E = Vec<T>::N;
    const int tid = threadIdx.x, lane = tid & 63;
    const int q = blockIdx.x / C, c = blockIdx.x % C;
    const int64_t nvec = V / E;
    const int64_t v0 = (int64_t)c * vpc;
    const int64_t v1 = v0 + vpc < nvec ? v0 + vpc : nvec;
    const bool tail_owner = c == C - 1;
    bool failed = false;
    if (blockIdx.x == 0 && tid == 0) mark_path(header, kPathAcceptCluster);

    // raw 16-byte vectors of this workgroup's chunk of the current row pair
    uint4 rd[NV], rt[NV];
    auto load_row = [&](int64_t row) {
        const T* dr = d + row * ldd;
        const T* tr = t + row * ldt;
        // lanes past the chunk re-read its last vector (never used; no chunk
        // is empty): a load under a lane condition merges with the register's
        // old value, and that merge waits for each load as it is issued
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            int64_t idx = v0 + tid + (int64_t)j * kCThreads;
            idx = idx < v1 ? idx : v1 - 1;
            rd[j] = *reinterpret_cast<const uint4*>(dr + idx * E);
            rt[j] = *reinterpret_cast<const uint4*>(tr + idx * E);
        }
    };
    // Rows after the first are claimed from a shared counter, so that clusters
    // that run faster (their workgroups are older on their CUs) take more of
    // them.  Member 0 claims the next row while this one loads; the index
    // travels to the other members with this row's statistics.
    uint32_t iter = 0;
    int64_t row = q;
    while (row < N) {
        const T* dr = d + row * ldd;
        const T* tr = t + row * ldt;
        load_row(row);
        uint32_t claim = 0;
        if (c == 0 && tid == 0) claim = __hip_atomic_fetch_add(&header[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // pass 1: running (max, sum) of this thread's elements
        float md = -INFINITY, sd = 0.f, mt = -INFINITY, st = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (v0 + tid + (int64_t)j * kCThreads < v1) {
                float xd[E], xt[E];
                unpack16<T>(rd[j], xd);
                unpack16<T>(rt[j], xt);
                fold<E>(md, sd, xd);
                fold<E>(mt, st, xt);
            }
        }
        if (tail_owner)
            for (int64_t v = nvec * E + tid; v < V; v += kCThreads) {
                float xd[1] = {load_elem(dr, v)}, xt[1] = {load_elem(tr, v)};
                fold<1>(md, sd, xd);
                fold<1>(mt, st, xt);
            }
        float Md = md, Sd = sd, Mt = mt, St = st;
        block_merge<kCThreads>(Md, Sd, lds);
        block_merge<kCThreads>(Mt, St, lds);

        if (C > 1) {  // meet the other chunks of this row
            const uint32_t tag = iter + 1;
            uint64_t* slot = stats + (((int64_t)q * 2 + (iter & 1)) * C) * 4;
            uint64_t* nslot = nexts + (int64_t)q * 2 + (iter & 1);
            if (tid == 0) {
                if (c == 0)
                    __hip_atomic_store(nslot, ((uint64_t)tag << 32) | (uint64_t)(uint32_t)(n_clusters + claim),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot + c * 4 + 0, tagged(tag, Md), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot + c * 4 + 1, tagged(tag, Sd), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot + c * 4 + 2, tagged(tag, Mt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot + c * 4 + 3, tagged(tag, St), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid < 64) {
                uint64_t w = tagged(tag, 0.f), nw = 0;
                bool ok = false;
                for (int spin = 0; spin < spin_limit && !failed; ++spin) {
                    w = lane < 4 * C ? __hip_atomic_load(slot + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                     : tagged(tag, 0.f);
                    nw = __hip_atomic_load(nslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = __all((uint32_t)(w >> 32) == tag && (uint32_t)(nw >> 32) == tag);
                    if (ok) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                if (!ok) failed = true;
                if (tid == 0) next_row = ok ? (int64_t)(uint32_t)nw : N;  // a lost member ends the cluster
                const float val = __uint_as_float((uint32_t)w);
                float M1 = -INFINITY, S1 = 0.f, M2 = -INFINITY, S2 = 0.f;  // chunks merged in order 0..C-1
                for (int k = 0; k < C; ++k) {
                    merge(M1, S1, __shfl(val, 4 * k), __shfl(val, 4 * k + 1));
                    merge(M2, S2, __shfl(val, 4 * k + 2), __shfl(val, 4 * k + 3));
                }
                if (tid == 0) {
                    rowstat[0] = failed ? __builtin_nanf("") : M1, rowstat[1] = S1;
                    rowstat[2] = M2, rowstat[3] = S2;
                    if (failed) mark_gave_up(header);
                }
            }
            __syncthreads();
            Md = rowstat[0], Sd = rowstat[1], Mt = rowstat[2], St = rowstat[3];
        } else {
            if (tid == 0) next_row = n_clusters + claim;
        }

        // pass 2: |p - q| with the normaliser folded into the exponent.  The raw
        // words go through an empty asm so that only they stay live across
        // the exchange, not their pass-1 conversions.
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            asm volatile("" : "+v"(rd[j].x), "+v"(rd[j].y), "+v"(rd[j].z), "+v"(rd[j].w));
            asm volatile("" : "+v"(rt[j].x), "+v"(rt[j].y), "+v"(rt[j].z), "+v"(rt[j].w));
        }
        const float cd = Md * kLog2e + __builtin_amdgcn_logf(Sd);
        const float ct = Mt * kLog2e + __builtin_amdgcn_logf(St);
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (v0 + tid + (int64_t)j * kCThreads < v1) {
                float xd[E], xt[E];
                unpack16<T>(rd[j], xd);
                unpack16<T>(rt[j], xt);
#pragma unroll
                for (int e = 0; e < E; ++e) acc += fabsf(exp_shifted(xd[e], cd) - exp_shifted(xt[e], ct));
            }
        }
        if (tail_owner)
            for (int64_t v = nvec * E + tid; v < V; v += kCThreads)
                acc += fabsf(exp_shifted(load_elem(dr, v), cd) - exp_shifted(load_elem(tr, v), ct));
        acc = block_sum<kCThreads>(acc, lds);

        if (C == 1) {
            if (tid == 0) out[row] = 1.f - 0.5f * acc;
        } else if (tid < 64) {
            // the partial sums are tagged words too; a relaxed counter elects
            // the finisher, which waits for every tag (no fence needed)
            const uint32_t tag = iter + 1;
            uint64_t* part = parts + ((int64_t)q * 2 + (iter & 1)) * C;
            uint32_t old = 0;
            if (tid == 0) {
                __hip_atomic_store(part + c, tagged(tag, acc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __hip_atomic_fetch_add(&counters[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            old = __shfl(old, 0);
            if (old == (uint32_t)C * (iter + 1) - 1) {  // last chunk of this row in: finish it
                uint64_t w = tagged(tag, 0.f);
                bool ok = false;
                for (int spin = 0; spin < spin_limit; ++spin) {
                    w = lane < C ? __hip_atomic_load(part + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : tagged(tag, 0.f);
                    ok = __all((uint32_t)(w >> 32) == tag);
                    if (ok) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                const float val = __uint_as_float((uint32_t)w);
                float sum = 0.f;
                for (int k = 0; k < C; ++k) sum += __shfl(val, k);
                if (tid == 0) {
                    out[row] = ok ? 1.f - 0.5f * sum : __builtin_nanf("");
                    if (!ok) mark_gave_up(header);
                }
            }
        }
        __syncthreads();  // next_row is written before the statistics barrier or here
        row = next_row;
        ++iter;
        __syncthreads();  // next_row is rewritten next row
    }

    // leave: the last workgroup out clears slots and counters for the next call
    // (also with C == 1: the row counter header[2] is claimed from either way)
    {
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(&header[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = old == gridDim.x - 1;
        }
        __syncthreads();
        if (last_flag) {
            for (int64_t i = tid; i < (int64_t)n_clusters * 2 * C * 4; i += kCThreads)
                __hip_atomic_store(stats + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int64_t i = tid; i < (int64_t)n_clusters * 2 * C; i += kCThreads)
                __hip_atomic_store(parts + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int64_t i = tid; i < n_clusters; i += kCThreads)
                __hip_atomic_store(counters + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int64_t i = tid; i < (int64_t)n_clusters * 2; i += kCThreads)
                __hip_atomic_store(nexts + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) {
                __hip_atomic_store(&header[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&header[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <typename T, int NV>
const void* cluster_fn() {
    return reinterpret_cast<const void*>(&accept_rate_cluster<T, NV>);
}

template <typename T>
const void* cluster_fn_nv(int nv) {
    static_assert(kCMaxVec == 10, "one instantiation per vector count");
    switch (nv) {
        case 1: return cluster_fn<T, 1>();
        case 2: return cluster_fn<T, 2>();
        case 3: return cluster_fn<T, 3>();
        case 4: return cluster_fn<T, 4>();
        case 5: return cluster_fn<T, 5>();
        case 6: return cluster_fn<T, 6>();
        case 7: return cluster_fn<T, 7>();
        case 8: return cluster_fn<T, 8>();
        case 9: return cluster_fn<T, 9>();
        default: return cluster_fn<T, 10>();
    }
}

int device_cus_ar() {
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

struct ClusterPlan {
    int C = 0, nv = 0, n_clusters = 0;
    int64_t vpc = 0;
    const void* fn = nullptr;
};

// Cluster shape for a row of V elements (nvec 16-byte vectors), or C == 0 if
// the rows do not fit the register budget.
template <typename T>
ClusterPlan plan_cluster(int64_t N, int64_t V) {
    ClusterPlan p;
    constexpr int E = Vec<T>::N;
    const int64_t nvec = V / E;
    if (nvec == 0) return p;  // rows shorter than one vector: the row kernel
    const int64_t per_wg = (int64_t)kCThreads * kCMaxVec;
    const int64_t C = (nvec + per_wg - 1) / per_wg;
    if (C > kCMaxCluster) return p;
    // no chunk is empty: (C - 1) ceil(nvec / C) < nvec because C (C - 1) < nvec
    const int64_t vpc = (nvec + C - 1) / C;
    const int nv = (int)((vpc + kCThreads - 1) / kCThreads);
    const void* fn = cluster_fn_nv<T>(nv < 1 ? 1 : nv);
    const int cus = device_cus_ar();
    int per_cu = 0;
    if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kCThreads, 0) != hipSuccess ||
        per_cu < 1)
        return p;
    const int64_t capacity = (int64_t)cus * per_cu;  // workgroups resident at once
    int64_t n_clusters = capacity / C;
    if (n_clusters > N) n_clusters = N;
    if (n_clusters < 1) return p;
    p.C = (int)C;
    p.nv = nv < 1 ? 1 : nv;
    p.vpc = vpc;
    p.n_clusters = (int)n_clusters;
    p.fn = fn;
    return p;
}

size_t cluster_workspace(int64_t N, int64_t V) {
    // sized for the largest cluster count any device could use
    (void)V;
    const int64_t max_clusters = N < 4096 ? N : 4096;
    // per cluster: statistics slots, partial-sum slots, a counter and the two
    // next-row words (with alignment slack)
    return kCHeader + (size_t)max_clusters * (2 * kCMaxCluster * 4 * 8 + 2 * kCMaxCluster * 8 + 4 + 252);
}

template <typename T>
hipError_t launch_typed(int64_t N, int64_t V, const void* d, int64_t ldd, const void* t, int64_t ldt, float* out,
                        void* ws, hipStream_t stream) {
    const bool vec = ((uintptr_t)d % 16 == 0) && ((uintptr_t)t % 16 == 0) && ((ldd * sizeof(T)) % 16 == 0) &&
                     ((ldt * sizeof(T)) % 16 == 0);
    const T* dp = static_cast<const T*>(d);
    const T* tp = static_cast<const T*>(t);
    if (vec && ws != nullptr) {
        const ClusterPlan p = plan_cluster<T>(N, V);
        if (p.C > 0 && (size_t)p.n_clusters <= (N < 4096 ? (size_t)N : (size_t)4096)) {
            char* w = static_cast<char*>(ws);
            uint32_t* header = reinterpret_cast<uint32_t*>(w);
            uint64_t* stats = reinterpret_cast<uint64_t*>(w + kCHeader);
            uint64_t* parts = reinterpret_cast<uint64_t*>(w + kCHeader + (size_t)p.n_clusters * 2 * p.C * 4 * 8);
            uint32_t* counters = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(parts) +
                                                             (size_t)p.n_clusters * 2 * p.C * 8);
            // the claimed next rows: two tagged words per cluster (inside the
            // per-cluster slack of cluster_workspace)
            uint64_t* nexts = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(counters) +
                                                          ((size_t)p.n_clusters * 4 + 7) / 8 * 8);
            int64_t NN = N, VV = V, vpc = p.vpc, ld1 = ldd, ld2 = ldt;
            int C = p.C, nc = p.n_clusters;
            int lim = wait_limit(kCSpinLimit);
            void* args[] = {&NN,  &VV,    &C,    &nc,       &vpc,  &dp,    &ld1,   &tp,
                            &ld2, &out,   &stats, &parts,   &counters, &nexts, &header, &lim};
            // at most the resident capacity: all workgroups of a cluster run together
            return hipLaunchKernel(p.fn, dim3((uint32_t)(p.n_clusters * p.C)), dim3(kCThreads), args, 0, stream);
        }
    }
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

size_t accept_rate_workspace(int64_t N, int64_t V) { return (cluster_workspace(N, V) + 255) / 256 * 256; }

hipError_t accept_rate_launch(int64_t N, int64_t V, int dtype, const void* d, int64_t ldd, const void* t,
                              int64_t ldt, float* out, void* ws, hipStream_t stream) {
    if (dtype == kBF16) return launch_typed<bf16_t>(N, V, d, ldd, t, ldt, out, ws, stream);
    return launch_typed<float>(N, V, d, ldd, t, ldt, out, ws, stream);
}

}  // namespace dspark
