// Hardware-aware prefix scheduler, Algorithm 1 of the DSpark paper as shown
// in "基于 DSpark 的投机解码训练框架原理与实现" (wangjunjian.com), section 3.3:
// sort the (request, position) pairs by survival a_{r,j} = prod_{i<=j} c_{r,i}
// in descending order, then scan greedily, accepting pairs while the
// throughput Theta = tau * SPS(Btok) improves and stopping at the first pair
// that does not improve it.
//
// One workgroup does the whole schedule (it is latency-bound: 4096 pairs in
// the training-width workload):
//   1. survivals as binary32 left-to-right products, one thread per request;
//      each pair's value is its complemented orderable survival, so an
//      ascending order of values is survival descending;
//   2. with every confidence in [0, 1] a product never grows, so each
//      request's run of values is already ascending: the global order is a
//      stable merge of the B runs (ties stay in request and position order).
//      The runs are merged pairwise in LDS, level by level, each thread
//      writing a few consecutive outputs after one binary search (merge
//      path).  If some run is not ascending (a confidence above 1), the merge
//      starts from runs of one pair instead: a plain merge sort, same order;
//   3. Theta for every prefix of the sorted list from a binary64 prefix sum.
//      When every summand is a multiple of 2^q and every partial sum stays
//      below 2^(q+53), binary64 addition is exact in any order, so the
//      parallel scan equals the sequential running sum bit for bit.  Sorted
//      survivals at or above 2^(ceil(log2(B(1+gamma)+1)) - 30) satisfy this
//      (they are multiples of 2^(e-23) and tau <= B(1+gamma)); the scan
//      covers that leading run in parallel and one wave finishes any
//      remaining pairs in sorted order, 64 at a time from registers;
//   4. the stop is the first prefix whose Theta does not exceed its
//      predecessor's (or the table's end); prefix lengths count the accepted
//      pairs per request in LDS.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kNT = 1024;
constexpr int kMaxPairs = 8192;
constexpr int kPer = kMaxPairs / kNT;  // sorted positions owned by each thread

__device__ __forceinline__ float val_survival(uint32_t v) { return from_orderable(~v); }

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int o) {
    const uint32_t lo = __shfl_up((uint32_t)v, o), hi = __shfl_up((uint32_t)(v >> 32), o);
    return ((uint64_t)hi << 32) | lo;
}

// Exclusive prefix sum of one value per thread across the workgroup, and the
// total (every thread gets both).
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* wsum, T& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    T off = incl - v, tot = 0;
    for (int w = 0; w < kNT / 64; ++w) {
        if (w < wave) off += wsum[w];
        tot += wsum[w];
    }
    total = tot;
    return off;
}

__global__ __launch_bounds__(kNT) void prefix_schedule_kernel(int64_t B, int64_t gamma, const float* __restrict__ conf,
                                                              const double* __restrict__ sps, int64_t n_sps,
                                                              float exact_floor, int32_t* __restrict__ prefix_len,
                                                              float* __restrict__ surv_out,
                                                              int32_t* __restrict__ order_out,
                                                              double* __restrict__ theta_out,
                                                              int32_t* __restrict__ nsel_out) {
    __shared__ uint32_t vals[2][kMaxPairs];  // ~orderable(survival): ascending = survival descending
    __shared__ uint16_t pids[2][kMaxPairs];  // pair id r * gamma + j of each value
    __shared__ double wsum[2 * kNT / 64];
    __shared__ uint32_t wpar[kNT / 64];
    __shared__ int stop_pos, n_exact, unsorted;
    __shared__ double tail_theta;
    __shared__ int tail_nsel, tail_mode;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)(B * gamma);
    const int g = (int)gamma;
    // Thread t owns sorted positions first+1 .. first+kPer.  Their table
    // entries (and the one before) do not depend on the sort: fetch them now.
    const int first = tid * kPer;
    double spv[kPer + 1];
#pragma unroll
    for (int q = 0; q <= kPer; ++q) {
        const int64_t i = B + first - 1 + q;
        spv[q] = i < n_sps ? sps[i] : 0.0;
    }

    if (tid == 0) stop_pos = 0x7fffffff, n_exact = 0, unsorted = 0;
    __syncthreads();
    if (g > 0) {
        // One thread per request, left to right (the same association as
        // the sequential product); the confidences come straight from
        // global memory, eight independent loads at a time.
        for (int r = tid; r < (int)B; r += kNT) {
            float p = 1.f;
            uint32_t prev = 0;
            bool up = true;
            for (int j0 = 0; j0 < g; j0 += 8) {
                float c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = j0 + j < g ? conf[r * g + j0 + j] : 1.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (j0 + j < g) {
                        const int pid = r * g + j0 + j;
                        p = p * c[j];
                        const uint32_t v = ~orderable(p);
                        up = up && v >= prev;
                        prev = v;
                        vals[0][pid] = v;
                        pids[0][pid] = (uint16_t)pid;
                    }
                }
            }
            if (!up) unsorted = 1;
        }
    }
    __syncthreads();
    if (surv_out)  // the survival is recovered exactly from its key
        for (int i = tid; i < n; i += kNT) surv_out[i] = val_survival(vals[0][i]);

    // Merge levels: runs of m pairs merged pairwise, ping-ponging between the
    // buffers.  The merge is stable (on equal values the left run goes
    // first), and every pair id of a left run is below every pair id of its
    // right run, so sorting the values gives the order (survival desc,
    // request asc, position asc).  A thread writes kc consecutive outputs: a
    // binary search finds how many of the first outputs of its merged run come
    // from the left run, then it merges forward with both run heads in
    // registers.
    const int kc = (n + kNT - 1) / kNT;
    int src = 0;
    for (int m = unsorted ? 1 : g; m > 0 && m < n; m *= 2) {
        const uint32_t* a = vals[src];
        const uint16_t* ai = pids[src];
        uint32_t* d = vals[src ^ 1];
        uint16_t* di = pids[src ^ 1];
        const int o0 = tid * kc;
        if (o0 < n) {
            int s0 = (o0 / (2 * m)) * (2 * m);
            int mid = s0 + m < n ? s0 + m : n, end = s0 + 2 * m < n ? s0 + 2 * m : n;
            const int dg = o0 - s0;
            int lo = dg - (end - mid) > 0 ? dg - (end - mid) : 0;
            int hi = dg < mid - s0 ? dg : mid - s0;
            while (lo < hi) {
                const int i = (lo + hi) >> 1;
                if (a[s0 + i] <= a[mid + dg - i - 1]) lo = i + 1;
                else hi = i;
            }
            int ia = s0 + lo, ib = mid + dg - lo;
            uint32_t va = ia < mid ? a[ia] : 0u, vb = ib < end ? a[ib] : 0u;
            for (int k = 0; k < kc && o0 + k < n; ++k) {
                const int o = o0 + k;
                if (o == end) {  // the next merged run starts
                    s0 = end;
                    mid = s0 + m < n ? s0 + m : n;
                    end = s0 + 2 * m < n ? s0 + 2 * m : n;
                    ia = s0;
                    ib = mid;
                    va = ia < mid ? a[ia] : 0u;
                    vb = ib < end ? a[ib] : 0u;
                }
                if (ia < mid && (ib >= end || va <= vb)) {
                    d[o] = va;
                    di[o] = ai[ia];
                    ++ia;
                    va = ia < mid ? a[ia] : 0u;
                } else {
                    d[o] = vb;
                    di[o] = ai[ib];
                    ++ib;
                    vb = ib < end ? a[ib] : 0u;
                }
            }
        }
        __syncthreads();
        src ^= 1;
    }
    const uint32_t* keys = vals[src];
    const uint16_t* ids = pids[src];
    int* counts = reinterpret_cast<int*>(vals[src ^ 1]);  // per-request tallies after the sort

    // Positions p = 1..n_lim may be accepted (the batch B + p must be in the table).
    const int n_lim = (int)((n_sps - B) < (int64_t)n ? (n_sps - B) : (int64_t)n);
    int my_ex = 0;
    for (int i = tid; i < n; i += kNT) my_ex += val_survival(keys[i]) >= exact_floor ? 1 : 0;
    for (int o = 32; o > 0; o >>= 1) my_ex += __shfl_xor(my_ex, o);
    if (lane == 0 && my_ex) atomicAdd(&n_exact, my_ex);
    if (order_out)
        for (int i = tid; i < n; i += kNT) order_out[i] = (int32_t)ids[i];
    for (int r = tid; r < (int)B; r += kNT) counts[r] = 0;
    __syncthreads();
    // Leading run of sorted survivals for which the parallel sum is exact.
    const int P = n_exact < n_lim ? n_exact : n_lim;

    // tau over positions 1..P: binary64 prefix sums (exact, see above).
    // inc[q] is the survival of an owned position p <= P.
    double inc[kPer];
    double local = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        inc[q] = (first + q < P) ? (double)val_survival(keys[first + q]) : 0.0;
        local += inc[q];
    }
    double S = 0.0;
    const double offset = block_exclusive_scan(local, wsum, S);
    const double Bd = (double)B;
    const double tauP = Bd + S;  // tau after position P

    // Theta over the exact run and the first position that does not improve
    {
        double tau_prev = Bd + offset;  // tau after position first (first <= P)
        double th_prev = tau_prev * spv[0];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = first + q + 1;
            if (p > P) break;
            const double tau = tau_prev + inc[q];
            const double th = tau * spv[q + 1];
            if (!(th > th_prev)) {
                atomicMin(&stop_pos, p);
                break;
            }
            tau_prev = tau;
            th_prev = th;
        }
    }
    __syncthreads();

    // Past P (survivals below the exact floor), tau stays in tauP's binade
    // [2^e, 2^(e+1)) as long as it grows by less than the distance to its
    // top.  There tau = u T with an integer T, u = 2^(e-52), and every
    // binary64 sum is u (T + rne(A)), A = a / u: the rounded increment is
    // floor(A) or floor(A) + 1 by the fraction of A, and at a tie (fraction
    // exactly 1/2) the one that makes T even.  So the running sum needs only
    // the parity of T before each tie: after a tie T is even, elsewhere the
    // parity flips with each odd increment -- a segmented XOR scan.  Then an
    // exact prefix sum of the increments (integers below 2^40 in binary64)
    // gives tau at every position at once, equal to the sequential running
    // sum.  A binade crossing or a non-finite value sends the tail to the
    // one-wave sequential finish instead.  inc[q] becomes the rounded
    // increment of an owned position p > P.  Skipped when the scan already
    // stopped inside the exact run.
    const bool need_tail = stop_pos == 0x7fffffff && P < n_lim;  // workgroup-uniform
    double u = 0.0, roff = 0.0;
    bool tail_ok = true;
    if (need_tail) {
        int ebin = 0;
        (void)frexp(tauP, &ebin);  // tauP = f 2^ebin, f in [0.5, 1)
        u = ldexp(1.0, ebin - 53);
        const double inv_u = ldexp(1.0, 53 - ebin);
        uint32_t tiemask = 0;  // owned positions with a tie
        uint32_t xr = 0;       // parity of the odd increments since the last owned tie
        int bad = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = first + q + 1;
            if (p > P && p <= n_lim) {
                const double A = (double)val_survival(keys[p - 1]) * inv_u;
                const double fl = floor(A), fr = A - fl;
                bad |= !(A >= 0.0 && A < 0x1p40) ? 1 : 0;
                const bool tie = fr == 0.5;
                inc[q] = fl + (fr > 0.5 ? 1.0 : 0.0);  // a tie's increment is settled below
                const uint32_t odd = (uint32_t)((uint64_t)fl & 1) ^ (fr > 0.5 ? 1u : 0u);
                tiemask |= tie ? (1u << q) : 0u;
                xr = tie ? 0u : xr ^ odd;
            }
        }
        // exclusive segmented scan of (parity, has tie) over threads in position order
        uint32_t x = xr, t = tiemask ? 1u : 0u;
        for (int o = 1; o < 64; o <<= 1) {  // inclusive within the wave
            const uint32_t xo = __shfl_up(x, o), to = __shfl_up(t, o);
            if (lane >= o) {
                x = t ? x : (xo ^ x);
                t = t | to;
            }
        }
        if (lane == 63) wpar[wave] = (x << 1) | t;
        const uint32_t xe = __shfl_up(x, 1), te = __shfl_up(t, 1);  // exclusive within the wave
        __syncthreads();
        uint32_t px = 0, pt = 0;  // waves before this one
        for (int w = 0; w < wave; ++w) {
            const uint32_t wx = wpar[w] >> 1, wt = wpar[w] & 1u;
            px = wt ? wx : (px ^ wx);
            pt |= wt;
        }
        if (lane > 0) {
            px = te ? xe : (px ^ xe);
            pt |= te;
        }
        // parity of T before this thread's first tail position
        uint32_t e = pt ? px : ((uint32_t)((uint64_t)(tauP * inv_u) & 1) ^ px);
        double rloc = 0.0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = first + q + 1;
            if (p > P && p <= n_lim) {
                if ((tiemask >> q) & 1u) {
                    const double fl = inc[q];
                    const uint32_t odd = (e ^ (uint32_t)((uint64_t)fl & 1)) & 1u;
                    inc[q] = fl + (double)odd;  // T + increment is even
                    e = 0;
                } else {
                    e ^= (uint32_t)((uint64_t)inc[q] & 1);
                }
                rloc += inc[q];
            }
        }
        double Ktot = 0.0;
        roff = block_exclusive_scan(rloc, wsum + kNT / 64, Ktot);
        tail_ok = !__syncthreads_or(bad) && tauP + u * Ktot < ldexp(1.0, ebin);

        // Theta on past the exact run (every exact position improved)
        if (tail_ok) {
            double tau_prev = first <= P ? Bd + offset : tauP + u * roff;  // tau after position first
            double th_prev = tau_prev * spv[0];
            double kq = roff;
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int p = first + q + 1;
                if (p > n_lim) break;
                double tau;
                if (p <= P) {
                    tau = tau_prev + inc[q];
                } else {
                    kq += inc[q];
                    tau = tauP + u * kq;
                }
                const double th = tau * spv[q + 1];
                if (p > P && !(th > th_prev)) {
                    atomicMin(&stop_pos, p);
                    break;
                }
                tau_prev = tau;
                th_prev = th;
            }
        }
        __syncthreads();
    }

    if (wave == 0) {
        int nsel = 0, mode = 0;
        double theta = 0.0;
        if (stop_pos != 0x7fffffff) {
            nsel = stop_pos - 1;  // Theta filled by the owner of position nsel
        } else if (P == n_lim || tail_ok) {
            nsel = n_lim;
        } else {
            // sequential finish beyond the exact run, in sorted order: 64
            // positions per round in registers, walked with lane reads
            mode = 1;
            double tau = tauP;
            theta = tau * sps[B + P - 1];
            nsel = P;
            bool go = true;
            for (int base = P; base < n_lim && go; base += 64) {
                const int p = base + 1 + lane;
                const double av = p <= n_lim ? (double)val_survival(keys[p - 1]) : 0.0;
                const double sv = p <= n_lim ? sps[B + p - 1] : 0.0;
                for (int q = 0; q < 64; ++q) {
                    if (base + 1 + q > n_lim) {
                        go = false;
                        break;
                    }
                    const double t2 = tau + readlane_f64(av, q);
                    const double th = t2 * readlane_f64(sv, q);
                    if (!(th > theta)) {
                        go = false;
                        break;
                    }
                    tau = t2;
                    theta = th;
                    nsel = base + 1 + q;
                }
            }
        }
        if (lane == 0) tail_nsel = nsel, tail_theta = theta, tail_mode = mode;
    }
    __syncthreads();
    const int nsel = tail_nsel;
    if (tid == 0 && tail_mode && theta_out) *theta_out = tail_theta;
    if (!tail_mode && theta_out) {
        // the owner of position nsel recomputes Theta there
        if (nsel == 0) {
            if (tid == 0) *theta_out = Bd * spv[0];
        } else if (nsel > first && nsel <= first + kPer) {
            // (fixed trip counts with predicates keep inc[] in registers)
            double tau = Bd + offset, k = roff;
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int p = first + q + 1;
                if (p <= nsel && p <= P) tau += inc[q];
                if (p <= nsel && p > P) k += inc[q];
            }
            if (nsel > P) tau = tauP + u * k;
            double sp = spv[0];
#pragma unroll
            for (int q = 1; q <= kPer; ++q) sp = first + q == nsel ? spv[q] : sp;
            *theta_out = tau * sp;
        }
    }
    if (tid == 0 && nsel_out) *nsel_out = nsel;
    for (int i = tid; i < nsel; i += kNT) atomicAdd(&counts[(uint32_t)ids[i] / (uint32_t)g], 1);
    __syncthreads();
    for (int r = tid; r < (int)B; r += kNT) prefix_len[r] = counts[r];
}

}  // namespace

size_t prefix_schedule_workspace(int64_t, int64_t) { return 0; }

hipError_t prefix_schedule_launch(int64_t B, int64_t gamma, const float* conf, const double* sps, int64_t n_sps,
                                  int32_t* prefix_len, float* survival_out, int32_t* order_out, double* theta_out,
                                  int32_t* n_selected_out, void*, hipStream_t stream) {
    // exact_floor = 2^(ceil(log2(B(1+gamma)+1)) - 30)
    const uint64_t cap = (uint64_t)B * (uint64_t)(1 + gamma) + 1;
    int e = 0;
    while ((1ull << e) < cap) ++e;
    const float floor = ldexpf(1.f, e - 30);
    hipLaunchKernelGGL(prefix_schedule_kernel, dim3(1), dim3(kNT), 0, stream, B, gamma, conf, sps, n_sps, floor,
                       prefix_len, survival_out, order_out, theta_out, n_selected_out);
    return hipGetLastError();
}

}  // namespace dspark
