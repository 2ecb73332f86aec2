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
//      each pair becomes a 64-bit key (complemented orderable survival, pair
//      id) so an ascending sort gives survival descending, then request and
//      position ascending;
//   2. bitonic sort of the keys in LDS;
//   3. Theta for every prefix of the sorted list from a binary64 prefix sum.
//      When every summand is a multiple of 2^q and every partial sum stays
//      below 2^(q+53), binary64 addition is exact in any order, so the
//      parallel scan equals the sequential running sum bit for bit.  Sorted
//      survivals at or above 2^(ceil(log2(B(1+gamma)+1)) - 30) satisfy this
//      (they are multiples of 2^(e-23) and tau <= B(1+gamma)); the scan
//      covers that leading run in parallel and finishes any remaining pairs
//      with one thread in sorted order;
//   4. the stop is the first prefix whose Theta does not exceed its
//      predecessor's (or the table's end); prefix lengths count the accepted
//      pairs per request.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kNT = 1024;
constexpr int kMaxPairs = 8192;
constexpr int kPer = kMaxPairs / kNT;  // sorted positions owned by each thread

__device__ __forceinline__ float key_survival(uint64_t k) { return from_orderable(~(uint32_t)(k >> 32)); }

__global__ __launch_bounds__(kNT) void prefix_schedule_kernel(int64_t B, int64_t gamma, const float* __restrict__ conf,
                                                              const double* __restrict__ sps, int64_t n_sps,
                                                              float exact_floor, int32_t* __restrict__ prefix_len,
                                                              float* __restrict__ surv_out,
                                                              int32_t* __restrict__ order_out,
                                                              double* __restrict__ theta_out,
                                                              int32_t* __restrict__ nsel_out) {
    __shared__ uint64_t keys[kMaxPairs];
    __shared__ double wsum[kNT / 64];
    __shared__ int stop_pos, n_exact;
    __shared__ double tail_theta;
    __shared__ int tail_nsel, tail_mode;

    const int tid = threadIdx.x;
    const int n = (int)(B * gamma);
    int npow = 2;
    while (npow < n) npow <<= 1;

    for (int i = tid; i < npow; i += kNT) keys[i] = ~0ull;
    for (int64_t r = tid; r < B; r += kNT) prefix_len[r] = 0;
    if (tid == 0) stop_pos = 0x7fffffff, n_exact = 0;
    __syncthreads();
    for (int64_t r = tid; r < B; r += kNT) {
        float p = 1.f;
        for (int64_t j = 0; j < gamma; ++j) {
            const int64_t pid = r * gamma + j;
            p = p * conf[pid];
            if (surv_out) surv_out[pid] = p;
            keys[pid] = ((uint64_t)(~orderable(p)) << 32) | (uint64_t)pid;
        }
    }
    __syncthreads();

    for (int size = 2; size <= npow; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (npow >> 1); i += kNT) {
                const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint64_t a = keys[lo], b = keys[hi];
                if ((a > b) == up) keys[lo] = b, keys[hi] = a;
            }
            __syncthreads();
        }
    }

    // Positions p = 1..n_lim may be accepted (the batch B + p must be in the table).
    const int n_lim = (int)((n_sps - B) < (int64_t)n ? (n_sps - B) : (int64_t)n);
    // Leading run of sorted survivals for which the parallel sum is exact.
    int my_ex = 0;
    for (int i = tid * kPer; i < tid * kPer + kPer; ++i)
        if (i < n && key_survival(keys[i]) >= exact_floor) ++my_ex;
    if (my_ex) atomicAdd(&n_exact, my_ex);
    if (order_out)
        for (int i = tid; i < n; i += kNT) order_out[i] = (int32_t)(uint32_t)keys[i];
    __syncthreads();
    const int P = n_exact < n_lim ? n_exact : n_lim;

    // Binary64 prefix sums over positions 1..P; thread t owns positions
    // t*kPer+1 .. t*kPer+kPer.
    const int first = tid * kPer;  // 0-based sorted index of this thread's first position
    double a_loc[kPer];
    double local = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = first + q;
        a_loc[q] = (i < P) ? (double)key_survival(keys[i]) : 0.0;
        local += a_loc[q];
    }
    // exclusive scan of per-thread sums across the workgroup
    const int lane = tid & 63, wave = tid >> 6;
    double incl = local;
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    double offset = incl - local;
    for (int w = 0; w < wave; ++w) offset += wsum[w];

    const double Bd = (double)B;
    double tau_prev = Bd + offset;                                  // tau after position first
    double th_prev = first < P ? tau_prev * sps[B + first - 1] : 0.0;  // Theta after position first
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int p = first + q + 1;
        if (p <= P) {
            const double tau = tau_prev + a_loc[q];
            const double th = tau * sps[B + p - 1];
            if (!(th > th_prev)) {
                atomicMin(&stop_pos, p);
                break;
            }
            tau_prev = tau;
            th_prev = th;
        }
    }
    __syncthreads();

    if (tid == 0) {
        int nsel, mode = 0;
        double theta = 0.0;
        if (stop_pos != 0x7fffffff || P == n_lim) {
            nsel = stop_pos != 0x7fffffff ? stop_pos - 1 : P;  // Theta filled by the owner of position nsel
        } else {
            mode = 1;
            // sequential finish beyond the exact run
            double S = 0.0;
            for (int w = 0; w < kNT / 64; ++w) S += wsum[w];
            double tau = Bd + S;
            theta = tau * sps[B + P - 1];
            nsel = P;
            for (int p = P + 1; p <= n_lim; ++p) {
                const double t2 = tau + (double)key_survival(keys[p - 1]);
                const double th = t2 * sps[B + p - 1];
                if (!(th > theta)) break;
                tau = t2;
                theta = th;
                nsel = p;
            }
        }
        tail_nsel = nsel;
        tail_theta = theta;
        tail_mode = mode;
    }
    __syncthreads();
    const int nsel = tail_nsel;
    if (tid == 0 && tail_mode && theta_out) *theta_out = tail_theta;
    if (!tail_mode && theta_out) {
        // position nsel lies in the exact run; its owner recomputes Theta there
        if (nsel == 0) {
            if (tid == 0) *theta_out = Bd * sps[B - 1];
        } else if (nsel > first && nsel <= first + kPer) {
            double tau = Bd + offset;
            for (int q = 0; first + q + 1 <= nsel; ++q) tau += a_loc[q];
            *theta_out = tau * sps[B + nsel - 1];
        }
    }
    if (tid == 0 && nsel_out) *nsel_out = nsel;
    for (int i = tid; i < nsel; i += kNT) {
        const uint32_t pid = (uint32_t)keys[i];
        atomicAdd(&prefix_len[pid / (uint32_t)gamma], 1);
    }
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
