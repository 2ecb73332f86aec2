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
//      The runs are merged pairwise in LDS, level by level; each pair finds
//      its place in the merged run with one binary search in the other run
//      and moves there.  If some run is not ascending (a confidence outside
//      [0, 1]), the merge starts from runs of one pair instead: a plain merge
//      sort, same order;
//   3. Theta for every prefix of the sorted list from a binary64 prefix sum.
//      When every summand is a multiple of 2^q and every partial sum stays
//      below 2^(q+53), binary64 addition is exact in any order, so the
//      parallel scan equals the sequential running sum bit for bit.  Sorted
//      survivals at or above 2^(ceil(log2(B(1+gamma)+1)) - 30) satisfy this
//      (they are multiples of 2^(e-23) and tau <= B(1+gamma)); the scan
//      covers that leading run in parallel.  Past it the running sum stays
//      exact in parallel as integer multiples of one binary64 step (see the
//      tail below); only a sum that crosses a power of two, or a value that
//      is not finite, leaves the rest to one wave, pair by pair in sorted
//      order, 64 at a time from registers;
//   4. the stop is the first prefix whose Theta does not exceed its
//      predecessor's (or the table's end); prefix lengths count the accepted
//      pairs per request in LDS.
#include <type_traits>

#include "internal.h"

namespace dspark {
namespace {

constexpr int kNT = 1024;
constexpr int kMaxPairs = 8192;
constexpr int kPer = kMaxPairs / kNT;  // sorted positions owned by each thread
constexpr int kConfChunk = 16;         // confidences loaded together per request
#ifndef DSPARK_SORT_SCALE
#define DSPARK_SORT_SCALE 1
#endif
constexpr int kSortScale = DSPARK_SORT_SCALE;  // outputs per sorting thread, times the minimum
static_assert(kPer == 8, "the owned keys are read as two 16-byte loads");

__device__ __forceinline__ float val_survival(uint32_t v) { return from_orderable(~v); }

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Lowers *stop to the wave's first stopping position: threads own positions
// in lane order, so the lowest lane that stopped holds the wave's minimum and
// one atomic per wave suffices (with every lane's atomic, thousands of them
// serialise on the one LDS word).
__device__ __forceinline__ void wave_stop(int my_stop, int lane, int* stop) {
    const uint64_t b = __ballot(my_stop != 0x7fffffff);
    if (b != 0 && lane == __ffsll((unsigned long long)b) - 1) atomicMin(stop, my_stop);
}

// DPP moves between lanes (register to register, no LDS round trip): a
// shift right by n lanes within each row of 16 (lanes near the row's start
// read 0) and the two broadcasts that join rows (lane 15 of each row into
// the next, lane 31 into rows 2 and 3; rows outside the mask read 0).
constexpr int kDppRowShr = 0x110;  // + n, 1 <= n <= 15
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)b), hi = dpp_u32<CTRL, ROWS>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sums within each row of 16 lanes (a tree of additions).
template <typename T, typename Move>
__device__ __forceinline__ T row_incl_scan(T x, Move mv) {
    x += mv(x, std::integral_constant<int, kDppRowShr + 1>{});
    x += mv(x, std::integral_constant<int, kDppRowShr + 2>{});
    x += mv(x, std::integral_constant<int, kDppRowShr + 4>{});
    x += mv(x, std::integral_constant<int, kDppRowShr + 8>{});
    return x;
}
struct MoveF64 {
    template <int C>
    __device__ double operator()(double v, std::integral_constant<int, C>) const { return dpp_f64<C, 0xf>(v); }
};
struct MoveU32 {
    template <int C>
    __device__ uint32_t operator()(uint32_t v, std::integral_constant<int, C>) const { return dpp_u32<C, 0xf>(v); }
};

// Inclusive prefix sums over the wave's 64 lanes: the rows' own scans, then
// the rows joined (a tree of additions).
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
    x = row_incl_scan(x, MoveF64{});
    x += dpp_f64<kDppRowBcast15, 0xa>(x);
    x += dpp_f64<kDppRowBcast31, 0xc>(x);
    return x;
}

// Inclusive prefix sums over lanes 0..kNT/64-1 (row 0) of one value each.
__device__ __forceinline__ double wave_totals_scan(double ws) {
    static_assert(kNT / 64 == 16, "the wave totals fill one row of 16 lanes");
    return row_incl_scan(ws, MoveF64{});
}

// Exclusive prefix sum of one value per thread across the workgroup, and the
// total (every thread gets both).  The additions form a tree, so the result
// is the sequential running sum only where binary64 addition is exact in any
// order -- which is how the scheduler uses it.
__device__ __forceinline__ double block_exclusive_scan(double v, double* wsum, double& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double incl = wave_incl_scan_f64(v);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    const double ws = wave_totals_scan(lane < kNT / 64 ? wsum[lane] : 0.0);
    total = readlane_f64(ws, kNT / 64 - 1);
    return (wave > 0 ? readlane_f64(ws, wave - 1) : 0.0) + (incl - v);
}

// q(e) = floor(e / d) for 0 <= e < 2^13 and d >= 1, from a binary32
// reciprocal within one ulp: (e + 1/2) / d lies at least 1/(2d) from an
// integer, and the reciprocal's error and the product's rounding move it by
// less than (e + 1/2)/d * 2^-22 < 2^-9 / d.
struct DivSmall {
    float inv;
    __device__ explicit DivSmall(int d) : inv(__builtin_amdgcn_rcpf((float)d)) {}  // within 1 ulp
    __device__ int q(int e) const { return (int)(((float)e + 0.5f) * inv); }
};

// Sort key of a survival: the complemented orderable bits, so ascending
// keys are descending survivals.  -0 and +0 are equal survivals: the order
// uses the key of +0 for both, so their pairs stay in request order.
__device__ __forceinline__ uint32_t canon_key(uint32_t v) { return v == 0x80000000u ? 0x7fffffffu : v; }

constexpr int kPad = 16;  // slack after each key and id row: window reads may run a few entries past n
using KeyRows = uint32_t (*)[kMaxPairs + kPad];
using IdRows = uint16_t (*)[kMaxPairs + kPad];

// The two runs of one merge, first level: run A is request ra and run B
// request ra + 1 (rb addresses it, clamped to a real request), read from the
// transposed keys; pair ids follow from the position.
struct TransposedPair {
    const uint32_t* scr;
    int ts, g, ra, rb;
    __device__ uint32_t ka(int i) const { return canon_key(scr[(i < g ? i : g - 1) * ts + ra]); }
    __device__ uint32_t kb(int j) const { return canon_key(scr[(j < g ? j : g - 1) * ts + rb]); }
    // the pair id of A[i] or B[j]
    __device__ int code_a(int i) const { return ra * g + i; }
    __device__ int code_b(int j) const { return (ra + 1) * g + j; }
    __device__ uint16_t id_of(int c) const { return (uint16_t)c; }
};
// Later levels: run A at a[sa..], run B at a[sb..] (sb <= n), ids beside them.
// Reads past a run stay inside the padded row.
struct NaturalPair {
    const uint32_t* a;
    const uint16_t* ai;
    int sa, sb;
    __device__ uint32_t ka(int i) const { return a[sa + i]; }
    __device__ uint32_t kb(int j) const { return a[sb + j]; }
    // the row position of A[i] or B[j]; its pair id is read from there
    __device__ int code_a(int i) const { return sa + i; }
    __device__ int code_b(int j) const { return sb + j; }
    __device__ uint16_t id_of(int c) const { return ai[c]; }
};

template <int KC>
__device__ __forceinline__ void store_run(uint32_t* d, uint16_t* di, const uint32_t (&v)[KC], const uint16_t (&id)[KC]) {
    if constexpr (KC == 1) {
        d[0] = v[0];
        di[0] = id[0];
    } else if constexpr (KC == 2) {
        *reinterpret_cast<uint2*>(d) = make_uint2(v[0], v[1]);
        *reinterpret_cast<uint32_t*>(di) = (uint32_t)id[0] | ((uint32_t)id[1] << 16);
    } else {
#pragma unroll
        for (int k = 0; k < KC; k += 4) {
            *reinterpret_cast<uint4*>(d + k) = make_uint4(v[k], v[k + 1], v[k + 2], v[k + 3]);
            *reinterpret_cast<uint2*>(di + k) = make_uint2((uint32_t)id[k] | ((uint32_t)id[k + 1] << 16),
                                                           (uint32_t)id[k + 2] | ((uint32_t)id[k + 3] << 16));
        }
    }
}

// Outputs dg .. dg+KC-1 of the merge of sorted runs A (lenA >= 1 keys) and B
// (lenB keys), equal keys from A first (merge path): a binary search finds
// how many of the first dg outputs come from A, then the next KC keys of
// each run are read together.  Each candidate becomes one 64-bit value, key
// above its source code (a code of A is below every code of B, and codes
// rise along a run), so the values are distinct and their order is the
// merge order.  The elementwise minimum of the A window and the reversed B
// window holds the KC smallest (a bitonic sequence); half-cleaners sort it.
// The keys and pair ids go out with vector stores at d, di (outputs past the
// end of the merged run are don't-cares).
template <int KC, typename Pair>
__device__ __forceinline__ void merge_path(const Pair& P, int lenA, int lenB, int dg, uint32_t* d, uint16_t* di) {
    int lo = dg - lenB > 0 ? dg - lenB : 0;
    int hi = dg < lenA ? dg : lenA;
    while (lo < hi) {
        const int i = (lo + hi) >> 1;
        if (P.ka(i) <= P.kb(dg - i - 1)) lo = i + 1;
        else hi = i;
    }
    const int pa = lo, pb = dg - lo;
    uint64_t c[KC], cb[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const uint64_t va = ((uint64_t)P.ka(pa + k) << 32) | (uint32_t)P.code_a(pa + k);
        const uint64_t vb = ((uint64_t)P.kb(pb + k) << 32) | (uint32_t)P.code_b(pb + k);
        c[k] = pa + k < lenA ? va : ~0ull;
        cb[k] = pb + k < lenB ? vb : ~0ull;
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) c[k] = cb[KC - 1 - k] < c[k] ? cb[KC - 1 - k] : c[k];
#pragma unroll
    for (int h = KC / 2; h > 0; h >>= 1) {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            if ((k & h) == 0) {
                const uint64_t x = c[k], y = c[k + h];
                c[k] = y < x ? y : x;
                c[k + h] = y < x ? x : y;
            }
        }
    }
    uint32_t ov[KC];
    uint16_t oid[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        ov[k] = (uint32_t)(c[k] >> 32);
        const uint32_t code = (uint32_t)c[k];
        oid[k] = P.id_of((int)(code < (uint32_t)(kMaxPairs - 1) ? code : (uint32_t)(kMaxPairs - 1)));
    }
    store_run<KC>(d, di, ov, oid);
}

// Stable sort of the n pair keys (ascending; equal keys in pair-id order).
// Each level merges runs of m pairwise.  Every pair id of a left run is
// below every pair id of its right run and equal keys take the left run
// first, so the order of equal keys is pair-id order.  With 2m a multiple of
// KC, thread t writes the KC consecutive outputs t*KC.. of one merged run
// (merge_path); otherwise (odd gamma at the first level) each thread moves
// the pairs t, t + kNT, ..., each to its index in its own run plus the
// number of pairs of the other run that go before it (smaller keys, and
// equal ones too when it is in the right run), found by one binary search
// whose probes are plain loads feeding selects.
//
// The keys arrive transposed in vals[0] (pair (r, j) at j * ts + r).  The
// first level reads them there and, with sorted runs, merges requests 2k and
// 2k+1 (m = gamma); otherwise it only lays the pairs out in request-major
// order and the merge starts from runs of one.  The first level also writes
// the survival output, coalesced.  Returns the row holding the result.
template <int KC>
__device__ int sort_pairs(int n, int g, int B, int ts, bool runs_sorted, float* __restrict__ surv_out, KeyRows vals,
                          IdRows pids) {
    const int tid = threadIdx.x;
    const uint32_t* scr = vals[0];
    const DivSmall dg(g);
    if (surv_out) {
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const int e = tid + kNT * q;
            if (e < n) {
                const int r = dg.q(e);
                surv_out[e] = from_orderable(~scr[(e - r * g) * ts + r]);  // the exact survival, sign included
            }
        }
    }
    if (runs_sorted && (2 * g) % KC == 0) {
        const int o0 = tid * KC;
        if (o0 < n) {
            const int ra = DivSmall(2 * g).q(o0) * 2;
            const TransposedPair P{scr, ts, g, ra, ra + 1 < B ? ra + 1 : ra};
            merge_path<KC>(P, g, ra + 1 < B ? g : 0, o0 - ra * g, vals[1] + o0, pids[1] + o0);
        }
    } else {
        uint32_t x[KC];
        int cnt[KC], rq[KC], jq[KC];
        bool act[KC];
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const int e = tid + kNT * q;
            act[q] = e < n;
            rq[q] = act[q] ? dg.q(e) : 0;
            jq[q] = act[q] ? e - rq[q] * g : 0;
            x[q] = canon_key(scr[jq[q] * ts + rq[q]]);
            cnt[q] = 0;
        }
        if (runs_sorted && B > 1) {
            int top = 1;
            while (2 * top <= g) top *= 2;
            for (int st = top; st > 0; st >>= 1) {
#pragma unroll
                for (int q = 0; q < KC; ++q) {
                    const int sr = rq[q] ^ 1;
                    const bool right = (rq[q] & 1) != 0;
                    const int jn = cnt[q] + st;
                    const bool ok = (sr < B) & (jn <= g);
                    const uint32_t y = canon_key(scr[(ok ? jn - 1 : 0) * ts + (ok ? sr : rq[q])]);
                    const bool take = ok & ((y < x[q]) | (right & (y == x[q])));
                    cnt[q] = take ? jn : cnt[q];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const int e = tid + kNT * q;
            if (act[q]) {
                const int pos = runs_sorted ? (rq[q] & ~1) * g + jq[q] + cnt[q] : e;
                vals[1][pos] = x[q];
                pids[1][pos] = (uint16_t)e;
            }
        }
    }
    __syncthreads();
    int src = 1;
    const int unit = runs_sorted ? g : 1;  // pairs per run after the first level
    const int o0 = tid * KC;
    const DivSmall du(unit);
    const int ou = du.q(o0);  // first output in units of the first level's runs (o0 < 2^13)
    int lvl = runs_sorted ? 1 : 0;
    for (int m = unit << lvl; m < n; m *= 2, ++lvl) {
        const uint32_t* a = vals[src];
        const uint16_t* ai = pids[src];
        uint32_t* d = vals[src ^ 1];
        uint16_t* di = pids[src ^ 1];
        if ((2 * m) % KC == 0) {
            if (o0 < n) {
                const int s0 = ((ou >> (lvl + 1)) << (lvl + 1)) * unit;  // floor(o0 / 2m) * 2m
                const int mid = s0 + m < n ? s0 + m : n;
                const int end = s0 + 2 * m < n ? s0 + 2 * m : n;
                const NaturalPair P{a, ai, s0, mid};
                merge_path<KC>(P, mid - s0, end - mid, o0 - s0, d + o0, di + o0);
            }
        } else {
            uint32_t x[KC];
            uint16_t id[KC];
            int cnt[KC], sb[KC], sl[KC], run[KC];
            bool right[KC];
#pragma unroll
            for (int q = 0; q < KC; ++q) {
                const int e = tid + kNT * q;
                const bool act = e < n;
                run[q] = du.q(e) >> lvl;
                const int s0 = run[q] * m;
                right[q] = (run[q] & 1) != 0;
                sb[q] = right[q] ? s0 - m : s0 + m;
                const int rest = n - sb[q];
                sl[q] = !act ? 0 : (right[q] ? m : (rest < m ? (rest > 0 ? rest : 0) : m));
                x[q] = a[act ? e : 0];
                id[q] = ai[act ? e : 0];
                cnt[q] = 0;
            }
            int top = 1;
            while (2 * top <= m) top *= 2;
            for (int st = top; st > 0; st >>= 1) {
#pragma unroll
                for (int q = 0; q < KC; ++q) {
                    const int jn = cnt[q] + st;
                    const bool ok = jn <= sl[q];
                    const uint32_t y = a[ok ? sb[q] + jn - 1 : 0];
                    const bool take = ok & ((y < x[q]) | (right[q] & (y == x[q])));
                    cnt[q] = take ? jn : cnt[q];
                }
            }
#pragma unroll
            for (int q = 0; q < KC; ++q) {
                const int e = tid + kNT * q;
                if (e < n) {
                    const int pos = (run[q] & ~1) * m + (e - run[q] * m) + cnt[q];
                    d[pos] = x[q];
                    di[pos] = id[q];
                }
            }
        }
        __syncthreads();
        src ^= 1;
    }
    return src;
}

__global__ __launch_bounds__(kNT) void prefix_schedule_kernel(int64_t B, int64_t gamma, const float* __restrict__ conf,
                                                              const double* __restrict__ sps, int64_t n_sps,
                                                              float exact_floor, int32_t* __restrict__ prefix_len,
                                                              float* __restrict__ surv_out,
                                                              int32_t* __restrict__ order_out,
                                                              double* __restrict__ theta_out,
                                                              int32_t* __restrict__ nsel_out) {
    __shared__ __align__(16) uint32_t vals[2][kMaxPairs + kPad];  // sort keys (canon_key): ascending = survival descending
    __shared__ __align__(16) uint16_t pids[2][kMaxPairs + kPad];  // pair id r * gamma + j of each key
    __shared__ double wsum[2 * kNT / 64];
    __shared__ uint32_t wpar[kNT / 64];
    __shared__ int stop_pos;
    __shared__ int wexact[kNT / 64];  // per wave: its positions in the exact run
    __shared__ int wunsorted[kNT / 64];  // per wave: some run of this wave's requests is not ascending
    __shared__ double tail_theta;
    __shared__ int tail_nsel;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)(B * gamma);
    const int g = (int)gamma;
    // Thread t owns sorted positions first+1 .. first+kPer.  Their table
    // entries (and the one before) do not depend on the sort: fetch them now
    // (B >= 1 and n_sps >= B, so the clamped index is always in the table).
    const int first = tid * kPer;
    double spv[kPer + 1];
#pragma unroll
    for (int q = 0; q <= kPer; ++q) {
        const int64_t i = B + first - 1 + q;
        const double v = sps[i < n_sps ? i : n_sps - 1];
        spv[q] = i < n_sps ? v : 0.0;
    }

    // (first read after the barrier that ends the survival phase)
    if (tid == 0) stop_pos = 0x7fffffff;
    // Keys of the request-major pairs, transposed: pair (r, j) sits at
    // j * ts + r, so a wave of consecutive requests stores to consecutive
    // words, and a wave of consecutive positions of one request (stride ts,
    // odd when it fits) reads from distinct banks.
    const int ts = (((int)B | 1) * g <= kMaxPairs) ? ((int)B | 1) : (int)B;
    uint32_t* scr = vals[0];
    bool all_up = true;
    // gamma a multiple of 4 (up to 16) and a 16-byte aligned array: each
    // product thread loads its own request's confidences with 16-byte loads,
    // so they skip the LDS round trip and its barrier
    const bool direct = ((uintptr_t)conf & 15) == 0 && g > 0 && g % 4 == 0 && g <= kConfChunk;
    if (direct) {
        for (int r = tid; r < (int)B; r += kNT) {
            float c[kConfChunk];
            const float4* cr = reinterpret_cast<const float4*>(conf + (int64_t)r * g);
#pragma unroll
            for (int j4 = 0; j4 < kConfChunk / 4; ++j4) {
                const float4 v = cr[4 * j4 < g ? j4 : 0];  // past gamma: any in-bounds vector, unused
                c[4 * j4] = v.x, c[4 * j4 + 1] = v.y, c[4 * j4 + 2] = v.z, c[4 * j4 + 3] = v.w;
            }
            float p = 1.f;
            uint32_t prev = 0;
            bool up = true;
#pragma unroll
            for (int j = 0; j < kConfChunk; ++j) {
                if (j < g) {
                    p = p * c[j];
                    const uint32_t v = ~orderable(p);
                    const uint32_t vc = canon_key(v);
                    up = up && vc >= prev;
                    prev = vc;
                    scr[j * ts + r] = v;
                }
            }
            all_up = all_up && up;
        }
    } else if (g > 0) {
        // The confidences, coalesced (four per thread per 16-byte load when
        // the array is 16-byte aligned), into the transposed layout...
        const bool vec = ((uintptr_t)conf & 15) == 0;
        const DivSmall dg(g);
        for (int e0 = 4 * tid; e0 < n; e0 += 4 * kNT) {
            float c[4];
            if (vec && e0 + 4 <= n) {
                const float4 v = *reinterpret_cast<const float4*>(conf + e0);
                c[0] = v.x, c[1] = v.y, c[2] = v.z, c[3] = v.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) c[k] = e0 + k < n ? conf[e0 + k] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = e0 + k;
                if (e < n) {
                    const int r = dg.q(e);
                    scr[(e - r * g) * ts + r] = __float_as_uint(c[k]);
                }
            }
        }
        __syncthreads();
        // ...then one thread per request, left to right (the same association
        // as the sequential product), each key replacing its confidence.  The
        // stored key keeps the sign of a zero survival (for the survival
        // output); the order uses the key of +0 for both zeros (see
        // canon_key).
        for (int r = tid; r < (int)B; r += kNT) {
            float p = 1.f;
            uint32_t prev = 0;
            bool up = true;
            for (int j0 = 0; j0 < g; j0 += kConfChunk) {
                float c[kConfChunk];
#pragma unroll
                for (int j = 0; j < kConfChunk; ++j) c[j] = __uint_as_float(scr[(j0 + j < g ? j0 + j : g - 1) * ts + r]);
#pragma unroll
                for (int j = 0; j < kConfChunk; ++j) {
                    if (j0 + j < g) {
                        p = p * c[j];
                        const uint32_t v = ~orderable(p);
                        const uint32_t vc = canon_key(v);
                        up = up && vc >= prev;
                        prev = vc;
                        scr[(j0 + j) * ts + r] = v;
                    }
                }
            }
            all_up = all_up && up;
        }
    }
    {
        const bool wave_unsorted = __ballot(!all_up) != 0;
        if (lane == 0) wunsorted[wave] = wave_unsorted ? 1 : 0;
    }
    __syncthreads();

    // Sort (see sort_pairs); kc pairs per thread at most.
    const int kc = (n + kNT - 1) / kNT;
    const bool runs_sorted = __ballot(lane < kNT / 64 && wunsorted[lane < kNT / 64 ? lane : 0] != 0) == 0;  // uniform
    int src = 1;
    if (g > 0) {
        const int kw = kc * kSortScale;
        if (kw <= 1) src = sort_pairs<1>(n, g, (int)B, ts, runs_sorted, surv_out, vals, pids);
        else if (kw <= 2) src = sort_pairs<2>(n, g, (int)B, ts, runs_sorted, surv_out, vals, pids);
        else if (kw <= 4) src = sort_pairs<4>(n, g, (int)B, ts, runs_sorted, surv_out, vals, pids);
        else src = sort_pairs<8>(n, g, (int)B, ts, runs_sorted, surv_out, vals, pids);
    }
    const uint32_t* keys = vals[src];
    const uint16_t* ids = pids[src];
    int* counts = reinterpret_cast<int*>(vals[src ^ 1]);  // per-request tallies after the sort

    // Positions p = 1..n_lim may be accepted (the batch B + p must be in the table).
    const int n_lim = (int)((n_sps - B) < (int64_t)n ? (n_sps - B) : (int64_t)n);
    // The keys of the owned positions, read once (two 16-byte loads).
    uint32_t kv[kPer];
    {
        const uint4 k0 = *reinterpret_cast<const uint4*>(keys + first);
        const uint4 k1 = *reinterpret_cast<const uint4*>(keys + first + 4);
        kv[0] = k0.x, kv[1] = k0.y, kv[2] = k0.z, kv[3] = k0.w;
        kv[4] = k1.x, kv[5] = k1.y, kv[6] = k1.z, kv[7] = k1.w;
    }
    if (order_out)
        for (int i = tid; i < n; i += kNT) order_out[i] = (int32_t)ids[i];
    // (the last merge level read this row before its barrier; the tallies
    // start after later barriers)
    for (int r = tid; r < (int)B; r += kNT) counts[r] = 0;
    // The exact run: positions 1..P, P = min(survivals at or above the floor,
    // n_lim); the sorted order puts those survivals first, so each thread
    // marks its own positions and the count rides on the scan's barrier.
    // tau over positions 1..P: binary64 prefix sums (exact, see above).
    // inc[q] is the survival of an owned position p <= P.
    double inc[kPer];
    double local = 0.0;
    int wave_ex = 0;  // the wave's positions in the exact run (uniform)
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const double a = (double)val_survival(kv[q]);
        const bool ex = first + q < n_lim && a >= (double)exact_floor;
        inc[q] = ex ? a : 0.0;
        local += inc[q];
        wave_ex += __popcll(__ballot(ex));
    }
    if (lane == 0) wexact[wave] = wave_ex;
    double S = 0.0;
    const double offset = block_exclusive_scan(local, wsum, S);
    // (written before the scan's barrier)
    const int P = (int)__builtin_amdgcn_readlane(
        (int)row_incl_scan((uint32_t)(lane < kNT / 64 ? wexact[lane] : 0), MoveU32{}), kNT / 64 - 1);
    const double Bd = (double)B;
    const double tauP = Bd + S;  // tau after position P

    // Theta over the exact run and the first position that does not improve
    {
        double tau_prev = Bd + offset;  // tau after position first (first <= P)
        double th_prev = tau_prev * spv[0];
        int my_stop = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = first + q + 1;
            if (p > P) break;
            const double tau = tau_prev + inc[q];
            const double th = tau * spv[q + 1];
            if (!(th > th_prev)) {
                my_stop = p;
                break;
            }
            tau_prev = tau;
            th_prev = th;
        }
        wave_stop(my_stop, lane, &stop_pos);
    }
    __syncthreads();

    // Past P (survivals below the exact floor), tau stays in tauP's binade
    // [2^e, 2^(e+1)) as long as it grows by less than the distance to its
    // top.  There tau = u T with an integer T, u = 2^(e-52), and every
    // binary64 sum is u (T + rne(A)), A = a / u: the rounded increment is
    // floor(A) or floor(A) + 1 by the fraction of A, and at a tie (fraction
    // exactly 1/2) the one that makes T even.  So the running sum needs only
    // the parity of T before each tie: after a tie T is even, elsewhere the
    // parity flips with each odd increment -- a segmented XOR scan, needed
    // only when some increment is a tie.  Then an exact prefix sum of the
    // increments (integers below 2^40 in binary64) gives tau at every
    // position at once, equal to the sequential running sum.  A binade
    // crossing or a non-finite value sends the tail to the one-wave
    // sequential finish instead.  inc[q] becomes the rounded increment of an
    // owned position p > P.  Skipped when the scan already stopped inside
    // the exact run.
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
        double rloc = 0.0;     // sum of the increments, ties counted at floor(A) for now
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = first + q + 1;
            if (p > P && p <= n_lim) {
                const double A = (double)val_survival(kv[q]) * inv_u;
                const double fl = floor(A), fr = A - fl;
                bad |= !(A >= 0.0 && A < 0x1p40) ? 1 : 0;
                const bool tie = fr == 0.5;
                inc[q] = fl + (fr > 0.5 ? 1.0 : 0.0);  // a tie's increment is settled below
                const uint32_t odd = (uint32_t)((uint64_t)fl & 1) ^ (fr > 0.5 ? 1u : 0u);
                tiemask |= tie ? (1u << q) : 0u;
                xr = tie ? 0u : xr ^ odd;
                rloc += inc[q];
            }
        }
        // One exchange: the wave sums of the increments, whether the wave
        // saw a non-finite value or a tie, and its parity summary (x = parity
        // of the odd increments after its last tie, t = it has a tie).
        const double incl = wave_incl_scan_f64(rloc);
        const bool wave_tie = __ballot(tiemask != 0) != 0;
        uint32_t x = xr, t = tiemask ? 1u : 0u;
        if (wave_tie) {  // inclusive segmented scan within the wave
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t xo = __shfl_up(x, o), to = __shfl_up(t, o);
                if (lane >= o) {
                    x = t ? x : (xo ^ x);
                    t = t | to;
                }
            }
        } else {  // no tie: the parity of all the wave's odd increments
            x = (uint32_t)__popcll(__ballot(xr != 0)) & 1u;
            t = 0;
        }
        const bool wave_bad = __ballot(bad != 0) != 0;
        if (lane == 63) {
            wsum[kNT / 64 + wave] = incl;
            wpar[wave] = (wave_bad ? 4u : 0u) | (x << 1) | t;
        }
        __syncthreads();
        // (integers below 2^53: exact in any order)
        const double ws = wave_totals_scan(lane < kNT / 64 ? wsum[kNT / 64 + lane] : 0.0);
        const uint32_t wp = lane < kNT / 64 ? wpar[lane] : 0u;
        double Ktot = readlane_f64(ws, kNT / 64 - 1);
        roff = (wave > 0 ? readlane_f64(ws, wave - 1) : 0.0) + (incl - rloc);
        const bool any_bad = __ballot((wp & 4u) != 0) != 0;
        const bool any_tie = __ballot((wp & 1u) != 0) != 0;
        if (any_tie) {
            // settle the ties from the parity of T before each one; then
            // the increments' prefix sums again
            if (!wave_tie) {  // this wave's lanes need their own exclusive parities
                x = xr;
                t = 0;
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t xo = __shfl_up(x, o);
                    if (lane >= o) x ^= xo;
                }
            }
            const uint32_t xe = __shfl_up(x, 1), te = __shfl_up(t, 1);  // exclusive within the wave
            uint32_t px = 0, pt = 0;  // waves before this one
            for (int w = 0; w < wave; ++w) {
                const uint32_t wx = (wpar[w] >> 1) & 1u, wt = wpar[w] & 1u;
                px = wt ? wx : (px ^ wx);
                pt |= wt;
            }
            if (lane > 0) {
                px = te ? xe : (px ^ xe);
                pt |= te;
            }
            // parity of T before this thread's first tail position
            uint32_t e = pt ? px : ((uint32_t)((uint64_t)(tauP * inv_u) & 1) ^ px);
            rloc = 0.0;
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
            roff = block_exclusive_scan(rloc, wsum, Ktot);  // (wsum[0..) is free again)
        }
        tail_ok = !any_bad && tauP + u * Ktot < ldexp(1.0, ebin);

        // Theta on past the exact run (stops inside it are recorded above;
        // a thread whose positions all lie inside it has nothing to do)
        if (tail_ok && first + kPer > P) {
            double tau_prev = first <= P ? Bd + offset : tauP + u * roff;  // tau after position first
            double th_prev = tau_prev * spv[0];
            double kq = roff;
            int my_stop = 0x7fffffff;
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
                    my_stop = p;
                    break;
                }
                tau_prev = tau;
                th_prev = th;
            }
            wave_stop(my_stop, lane, &stop_pos);
        }
    }
    __syncthreads();  // every stop is in

    int nsel = 0;
    bool seq = false;  // workgroup-uniform
    if (stop_pos != 0x7fffffff) {
        nsel = stop_pos - 1;  // Theta filled by the owner of position nsel
    } else if (P == n_lim || tail_ok) {
        nsel = n_lim;
    } else {
        seq = true;
    }
    if (seq) {
        if (wave == 0) {
            // sequential finish beyond the exact run, in sorted order: 64
            // positions per round in registers, walked with lane reads
            double tau = tauP;
            double theta = tau * sps[B + P - 1];
            int ns = P;
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
                    ns = base + 1 + q;
                }
            }
            if (lane == 0) tail_nsel = ns, tail_theta = theta;
        }
        __syncthreads();
        nsel = tail_nsel;
        if (tid == 0 && theta_out) *theta_out = tail_theta;
    }
    if (!seq && theta_out) {
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
    {
        const DivSmall dg(g > 0 ? g : 1);
        for (int i = tid; i < nsel; i += kNT) atomicAdd(&counts[dg.q(ids[i])], 1);
    }
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
