// Teacher-forced block bias with the joint training loss ("基于 DSpark 的投机解码
// 训练框架原理与实现", wangjunjian.com, section 7.2, the joint loss; the
// training loop applies the sequential head with the given previous tokens,
// section 3.2 and paper eq. 5 for the bias).
//
// With the previous tokens given, every position is independent:
//   d[p][v] = U[p][v] + W2[v] . W1[xp[p]]            (draft logits)
// and the loss needs, per position, logsumexp(d), d[y], and
// L1 = 1/2 sum_v |softmax(d)_v - softmax(t)_v|, which needs both row
// normalisers before it can be summed.  Both distributions sum to one, so
// L1 = 1 - sum_v min(p_v, q_v), and the min of two probabilities is the
// exponential of the smaller exponent: one exponential per row instead of
// two.  Five launches:
//   loss_stream<1>  a workgroup takes a 256-row vocabulary chunk, holds
//                   those W2 rows in registers as matrix-core A fragments and
//                   streams up to 1024 positions through them, 32 at a time:
//                   d on the matrix cores (bf16 in, fp32 accumulate), the U
//                   and t tiles and the embeddings W1[xp] staged through LDS
//                   with two blocks of loads in flight in registers; per
//                   position and chunk it writes (max, sum) of d and t;
//   loss_merge      per position: the chunk partials merged in a fixed order
//                   into logsumexp(d) and logsumexp(t), the target's logit
//                   d[y] = U[y] + W2[y] . W1[xp], and the confidence logit
//                   w . [h; W1[xp]] + b;
//   loss_stream<2>  the same stream again, summing min(p_d, p_t) per chunk;
//   loss_final      per position: L1, CE, c* = 1 - L1, conf, BCE and the
//                   position's weighted terms;
//   loss_reduce     one workgroup sums the terms over positions in a fixed
//                   order.
// W2 crosses HBM once per (chunk, position group) work item, U and t once
// per pass.  Every workspace word is written before it is read, so the
// workspace needs no clearing, and every reduction runs in a fixed order:
// repeated calls are bitwise identical.
#include <type_traits>

#include "block_loss.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRank = 256;          // Markov rank of the matrix-core tiles
constexpr int kSWaves = 8;          // waves per streaming workgroup, 32 vocabulary rows each
constexpr int kSThreads = 64 * kSWaves;
constexpr int kChunk = 32 * kSWaves;  // vocabulary rows per chunk (one work item's W2 rows)
constexpr int kBlk = 32;            // positions per block (one 32-wide MFMA tile)
constexpr int kGroupPos = 1024;     // positions per work item
constexpr int kRow = kRank + 8;     // LDS row stride (bf16) of E and of the U and t tiles (both 256 wide)
static_assert(kChunk == kRank && kSThreads == 2 * kBlk * 8, "16 threads per position, two 8-column pieces each");
constexpr int kReduceThreads = 1024;

constexpr uint32_t kNegInf2 = 0xff80ff80u;  // two bf16 -inf
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// e^(x - m) as 2^(x log2 e - m log2 e), the argument in one fused step; mk = m log2 e
__device__ __forceinline__ float exp_shift(float x, float mk) { return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -mk)); }

// (m, s) pairs of an online softmax normaliser: merge b into a.
__device__ __forceinline__ void merge_ms(float& m, float& s, float mb, float sb) {
    const float mm = fmaxf(m, mb);
    if (mm == -INFINITY) return;  // both empty
    s = s * __expf(m - mm) + sb * __expf(mb - mm);
    m = mm;
}

// One block's loads, held in registers until they are staged in LDS.  Thread
// t covers position t / 16 of the block and two pieces of 8 columns,
// 8 (t % 16) and 128 + 8 (t % 16): of the U and t tiles (vocabulary rows
// vt + ...) and of the embedding W1[xp] (rank elements).  So the 16 threads
// of a position read 256 contiguous bytes per load instruction, four whole
// 64-byte lines.  Positions past the end repeat the last
// one; rows past V read as bf16 -inf in both tiles, so they drop out of every
// max, exponential and sum without a test in the epilogue.
struct BlockRegs {
    u32x4_t u[2], t[2], e[2];
    float l0, l1;  // pass 2: logsumexp of d and t of the lane's position (lane % 32)
};

// The item's previous tokens (and in pass 2 its normalisers) sit in LDS, so
// no load here waits for another load.
struct ItemSide {
    int32_t x[kGroupPos];
    float a[kGroupPos], b[kGroupPos];  // pass 2: the two logsumexps
};

template <int PASS, bool VEC>
__device__ __forceinline__ void load_block(BlockRegs& r, const bf16_t* __restrict__ U, const bf16_t* __restrict__ T,
                                           const bf16_t* __restrict__ W1, const ItemSide& side, int64_t V,
                                           int64_t p_begin, int64_t pb, int64_t p_end, int64_t vt, int tid) {
    const int pl = tid >> 4, c0 = (tid & 15) * 8;
    const int64_t p = pb + pl < p_end ? pb + pl : p_end - 1;
    const int32_t x = side.x[p - p_begin];  // already made a valid row
    const u32x4_t* er = reinterpret_cast<const u32x4_t*>(W1 + (int64_t)x * kRank + c0);
    r.e[0] = er[0];
    r.e[1] = er[kRank / 2 / 8];
    const uint16_t* ur = reinterpret_cast<const uint16_t*>(U + p * V);
    const uint16_t* tr = reinterpret_cast<const uint16_t*>(T + p * V);
    const int64_t v = vt + c0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t vi = v + kChunk / 2 * i;
        if (VEC) {  // V % 8 == 0: a piece is wholly in or out
            const bool in = vi + 8 <= V;
            const int64_t vc = in ? vi : V - 8;  // out of range: an in-bounds read, replaced below
            const u32x4_t uw = *reinterpret_cast<const u32x4_t*>(ur + vc);
            const u32x4_t tw = *reinterpret_cast<const u32x4_t*>(tr + vc);
            const u32x4_t ninf = {kNegInf2, kNegInf2, kNegInf2, kNegInf2};
            r.u[i] = in ? uw : ninf;
            r.t[i] = in ? tw : ninf;
        } else {
            uint32_t wu[4], wt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t a = vi + 2 * j, b = a + 1;
                wu[j] = (a < V ? ur[a] : 0xff80u) | (b < V ? (uint32_t)ur[b] << 16 : 0xff800000u);
                wt[j] = (a < V ? tr[a] : 0xff80u) | (b < V ? (uint32_t)tr[b] << 16 : 0xff800000u);
            }
            r.u[i] = u32x4_t{wu[0], wu[1], wu[2], wu[3]};
            r.t[i] = u32x4_t{wt[0], wt[1], wt[2], wt[3]};
        }
    }
    const int lane = tid & 63;
    const int64_t q = (pb + (lane & 31) < p_end ? pb + (lane & 31) : p_end - 1) - p_begin;
    if (PASS == 2) r.l0 = side.a[q], r.l1 = side.b[q];
}

__device__ __forceinline__ void stage_block(const BlockRegs& r, uint16_t* E, uint16_t* Ut, uint16_t* Tt, int tid) {
    const int pl = tid >> 4, c0 = (tid & 15) * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        *reinterpret_cast<u32x4_t*>(E + pl * kRow + c0 + kRank / 2 * i) = r.e[i];
        *reinterpret_cast<u32x4_t*>(Ut + pl * kRow + c0 + kChunk / 2 * i) = r.u[i];
        *reinterpret_cast<u32x4_t*>(Tt + pl * kRow + c0 + kChunk / 2 * i) = r.t[i];
    }
}

// Persistent grid (at most one workgroup per compute unit), kSThreads
// threads.  The work is nchunk x nb blocks (nb = ceil(M / kBlk)), chunk
// major; workgroup g takes the contiguous share [g total / G, (g + 1) total
// / G), cut into items of one chunk and at most kGroupPos positions.
// PASS 1 writes the chunk's (max, sum) of d and t per position to stats
// [M][chunks][4]; PASS 2 reads lse [M][2] and writes the chunk's sum of
// min(p_d, p_t) to l1p [M][chunks].
template <int PASS, bool VEC>
__global__ __launch_bounds__(kSThreads) void loss_stream(int64_t M, int64_t V, int64_t nchunk,
                                                         const bf16_t* __restrict__ U, const bf16_t* __restrict__ T,
                                                         const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W2,
                                                         const int32_t* __restrict__ xp, float* __restrict__ stats,
                                                         const float* __restrict__ lse, float* __restrict__ l1p) {
    __shared__ __align__(16) uint16_t E_lds[2][kBlk * kRow];
    __shared__ __align__(16) uint16_t U_lds[2][kBlk * kRow];
    __shared__ __align__(16) uint16_t T_lds[2][kBlk * kRow];
    __shared__ float red[kSWaves][kBlk][4];
    __shared__ ItemSide side;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, row = lane & 31, half = lane >> 5;

    const int64_t nb = (M + kBlk - 1) / kBlk, total = nchunk * nb;
    const int64_t u_hi = total * (blockIdx.x + 1) / gridDim.x;
    for (int64_t u = total * blockIdx.x / gridDim.x; u < u_hi;) {  // workgroup-uniform
        const int64_t chunk = u / nb, b0 = u % nb;
        int64_t b1 = b0 + kGroupPos / kBlk < nb ? b0 + kGroupPos / kBlk : nb;
        b1 = b1 - b0 < u_hi - u ? b1 : b0 + (u_hi - u);
        u += b1 - b0;
        const int64_t vt = chunk * kChunk;
        const int64_t p_begin = b0 * kBlk;
        const int64_t p_end = b1 * kBlk < M ? b1 * kBlk : M;
        const int nblk = (int)(b1 - b0);

        // this wave's 32 W2 rows as A fragments: k-step s takes rank
        // elements 16 s + 8 half .. + 7 of row vt + 32 wave + row
        uint4 a[16];
        {
            int64_t v = vt + wave * 32 + row;
            v = v < V ? v : V - 1;  // clamped; its products are never used
            const uint4* src = reinterpret_cast<const uint4*>(W2 + v * kRank + half * 8);
#pragma unroll
            for (int s = 0; s < 16; ++s) a[s] = src[2 * s];
        }
        __syncthreads();  // the previous item is done with the LDS
        for (int i = tid; i < p_end - p_begin; i += kSThreads) {
            int32_t x = xp[p_begin + i];
            if (x < 0 || x >= V) x = 0;  // such a position's outputs are NaN; any row will do
            side.x[i] = x;
            if (PASS == 2) side.a[i] = lse[2 * (p_begin + i)], side.b[i] = lse[2 * (p_begin + i) + 1];
        }
        __syncthreads();
        BlockRegs rg[2];
        load_block<PASS, VEC>(rg[0], U, T, W1, side, V, p_begin, p_begin, p_end, vt, tid);
        load_block<PASS, VEC>(rg[1], U, T, W1, side, V, p_begin, p_begin + kBlk, p_end, vt, tid);
        stage_block(rg[0], E_lds[0], U_lds[0], T_lds[0], tid);
        float cur_l0 = rg[0].l0, cur_l1 = rg[0].l1;
        load_block<PASS, VEC>(rg[0], U, T, W1, side, V, p_begin, p_begin + 2 * kBlk, p_end, vt, tid);
        __syncthreads();

        // One block: SLOT holds block b; nr holds block b + 1 (in flight),
        // the other register set block b + 2.  The two sets swap roles from
        // block to block, so the loop is unrolled by two and each set is
        // named statically (selecting between them at run time would wait
        // for both).
        auto block = [&](auto slot_c, BlockRegs& nr, int b) {
            constexpr int slot = decltype(slot_c)::value;
            const int64_t pb = p_begin + (int64_t)b * kBlk;
            // d of this wave's 32 rows for the block's 32 positions
            f32x16_t acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const uint4 bw = *reinterpret_cast<const uint4*>(&E_lds[slot][row * kRow + s * 16 + half * 8]);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                              __builtin_bit_cast(bf16x8_t, bw), acc, 0, 0, 0);
            }
            // lane: position pb + row, vocabulary rows vt + 32 wave + 8 (r / 4) + 4 half + r % 4;
            // the U and t values stay packed (two per register) and are widened where used
            const uint16_t* ul = &U_lds[slot][row * kRow + wave * 32 + 4 * half];
            const uint16_t* tl = &T_lds[slot][row * kRow + wave * 32 + 4 * half];
            uint2 uu[4], tt[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uu[q] = *reinterpret_cast<const uint2*>(ul + 8 * q);
                tt[q] = *reinterpret_cast<const uint2*>(tl + 8 * q);
            }
            auto word = [](const uint2& w, int j) { return j < 2 ? w.x : w.y; };
            auto d_at = [&](int r) {  // rows past V: -inf (the U tile holds -inf there)
                const uint32_t w = word(uu[r / 4], r % 4);
                return ((r & 1) ? widen_hi(w) : widen_lo(w)) + acc[r];
            };
            auto t_at = [&](int r) {
                const uint32_t w = word(tt[r / 4], r % 4);
                return (r & 1) ? widen_hi(w) : widen_lo(w);
            };
            float o0, o1 = 0.f, o2 = 0.f, o3 = 0.f;
            if (PASS == 1) {
                float md = -INFINITY, mt = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) md = fmaxf(md, d_at(r)), mt = fmaxf(mt, t_at(r));
                // a lane whose rows are all -inf on one side sums zeros there (shift 0, not -inf)
                float sd = 0.f, st = 0.f;
                const float mdk = md > -INFINITY ? md * kLog2e : 0.f, mtk = mt > -INFINITY ? mt * kLog2e : 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) sd += exp_shift(d_at(r), mdk), st += exp_shift(t_at(r), mtk);
                const float m2 = __shfl_xor(md, 32), s2 = __shfl_xor(sd, 32);
                const float m3 = __shfl_xor(mt, 32), s3 = __shfl_xor(st, 32);
                merge_ms(md, sd, m2, s2);
                merge_ms(mt, st, m3, s3);
                o0 = md, o1 = sd, o2 = mt, o3 = st;
            } else {
                // sum of min(p_d, p_t): one exponential per row; a -inf logit is
                // probability 0 (rows past V: 0 on both sides)
                float sum = 0.f;
                const float l0k = cur_l0 * kLog2e, l1k = cur_l1 * kLog2e;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sum += __builtin_amdgcn_exp2f(fminf(fmaf(d_at(r), kLog2e, -l0k), fmaf(t_at(r), kLog2e, -l1k)));
                o0 = sum + __shfl_xor(sum, 32);
            }
            if (half == 0) {
                red[wave][row][0] = o0;
                if (PASS == 1) red[wave][row][1] = o1, red[wave][row][2] = o2, red[wave][row][3] = o3;
            }
            __syncthreads();  // red is complete; every wave is done with this slot
            if (PASS == 1 && tid < 2 * kBlk) {
                // the eight waves' (max, sum) pairs of one position and one side
                // (lanes 0-31: d, 32-63: t): the maximum first, then the
                // rescaled sums in wave order, all eight exponentials at once
                const int pl = tid & 31, q = (tid >> 5) * 2;
                float mw[kSWaves], sw[kSWaves];
#pragma unroll
                for (int w = 0; w < kSWaves; ++w) mw[w] = red[w][pl][q], sw[w] = red[w][pl][q + 1];
                float mm = mw[0];
#pragma unroll
                for (int w = 1; w < kSWaves; ++w) mm = fmaxf(mm, mw[w]);
                float ss = 0.f;
                if (mm > -INFINITY) {  // else every wave saw only -inf: an empty sum
#pragma unroll
                    for (int w = 0; w < kSWaves; ++w) ss += sw[w] * __expf(mw[w] - mm);
                }
                const float mt2 = __shfl_down(mm, 32), st2 = __shfl_down(ss, 32);
                if (tid < kBlk && pb + tid < p_end) {
                    float4 o;
                    o.x = mm, o.y = ss, o.z = mt2, o.w = st2;
                    reinterpret_cast<float4*>(stats)[(pb + tid) * nchunk + chunk] = o;
                }
            }
            if (PASS == 2 && tid < kBlk && pb + tid < p_end) {  // the eight waves, in order
                float t = red[0][tid][0];
                for (int w = 1; w < kSWaves; ++w) t += red[w][tid][0];
                l1p[(pb + tid) * nchunk + chunk] = t;
            }
            // block b + 1 into the other slot; its registers then take block
            // b + 3 (unconditionally: past the last block they re-read the last
            // position, in bounds and never used, which keeps the waits one
            // block deep)
            stage_block(nr, E_lds[slot ^ 1], U_lds[slot ^ 1], T_lds[slot ^ 1], tid);
            cur_l0 = nr.l0, cur_l1 = nr.l1;
            load_block<PASS, VEC>(nr, U, T, W1, side, V, p_begin, pb + 3 * kBlk, p_end, vt, tid);
            __syncthreads();  // slot b + 1 is staged; red may be rewritten
        };
        for (int b = 0; b < nblk; b += 2) {
            block(std::integral_constant<int, 0>{}, rg[1], b);
            if (b + 1 < nblk) block(std::integral_constant<int, 1>{}, rg[0], b + 1);
        }
    }
}

// grid M, 256 threads: lse [M][2] = (logsumexp d, logsumexp t) from the chunk
// partials, the target's draft logit dy [M] = U[y] + W2[y] . W1[xp] (rank
// kRank, one product per thread) and the confidence logit
// zc [M] = w . [h; W1[xp]] + b.
__global__ __launch_bounds__(256) void loss_merge(int64_t M, int64_t V, int64_t H, int64_t nchunk,
                                                  const float* __restrict__ stats, const bf16_t* __restrict__ U,
                                                  const bf16_t* __restrict__ h, const bf16_t* __restrict__ W1,
                                                  const bf16_t* __restrict__ W2, const bf16_t* __restrict__ w,
                                                  float b_conf, const int32_t* __restrict__ xp,
                                                  const int32_t* __restrict__ y, float* __restrict__ lse,
                                                  float* __restrict__ dy, float* __restrict__ zc) {
    static_assert(kRank == 256, "one rank element per thread");
    __shared__ float rm[256][4];
    __shared__ float rz[4], rd[4];
    const int64_t p = blockIdx.x;
    const int tid = threadIdx.x;
    float m1 = -INFINITY, s1 = 0.f, m2 = -INFINITY, s2 = 0.f;
    for (int64_t c = tid; c < nchunk; c += 256) {
        const float4 o = reinterpret_cast<const float4*>(stats)[p * nchunk + c];
        merge_ms(m1, s1, o.x, o.y);
        merge_ms(m2, s2, o.z, o.w);
    }
    rm[tid][0] = m1, rm[tid][1] = s1, rm[tid][2] = m2, rm[tid][3] = s2;
    int32_t x = xp[p], yy = y[p];
    if (x < 0 || x >= V) x = 0;
    if (yy < 0 || yy >= V) yy = 0;  // such a position's outputs are NaN; any row will do
    float z = 0.f;
    for (int64_t i = tid; i < H + kRank; i += 256)
        z += load_elem(w, i) * (i < H ? load_elem(h, p * H + i) : load_elem(W1, (int64_t)x * kRank + (i - H)));
    float d = load_elem(W2, (int64_t)yy * kRank + tid) * load_elem(W1, (int64_t)x * kRank + tid);
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o), d += __shfl_xor(d, o);
    if ((tid & 63) == 0) rz[tid >> 6] = z, rd[tid >> 6] = d;
    __syncthreads();
    for (int n = 128; n > 0; n >>= 1) {  // tree over threads, fixed order
        if (tid < n) {
            merge_ms(rm[tid][0], rm[tid][1], rm[tid + n][0], rm[tid + n][1]);
            merge_ms(rm[tid][2], rm[tid][3], rm[tid + n][2], rm[tid + n][3]);
        }
        __syncthreads();
    }
    if (tid == 0) {
        lse[2 * p] = rm[0][0] + __logf(rm[0][1]);
        lse[2 * p + 1] = rm[0][2] + __logf(rm[0][3]);
        dy[p] = load_elem(U, p * V + yy) + (((rd[0] + rd[1]) + rd[2]) + rd[3]);
        zc[p] = ((rz[0] + rz[1]) + rz[2]) + rz[3] + b_conf;
    }
}

// grid ceil(M / 4), 256 threads: one wave per position (the chunk partials
// summed lane-strided, then across the wave in a fixed order); per-position
// outputs and weighted terms [M][4].
__global__ __launch_bounds__(256) void loss_final(int64_t M, int64_t gamma, int64_t V, int64_t nchunk,
                                                  const float* __restrict__ l1p, const float* __restrict__ dy,
                                                  const float* __restrict__ lse, const float* __restrict__ zc,
                                                  const int32_t* __restrict__ xp, const int32_t* __restrict__ y,
                                                  const float* __restrict__ mask, float decay,
                                                  float* __restrict__ ce, float* __restrict__ l1,
                                                  float* __restrict__ conf, float* __restrict__ bce,
                                                  float* __restrict__ terms) {
    const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (p >= M) return;  // whole waves
    float s = 0.f;
    for (int64_t c = lane; c < nchunk; c += 64) s += l1p[p * nchunk + c];
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane != 0) return;
    const int32_t x = xp[p], yy = y[p];
    float4 tm;
    tm.x = tm.y = tm.z = tm.w = 0.f;
    if (x < 0 || x >= V || yy < 0 || yy >= V) {
        ce[p] = l1[p] = conf[p] = bce[p] = __builtin_nanf("");
    } else {
        // sum of min(p_d, p_t) = 1 - L1, kept in [0, 1] (rounding can put the
        // sum a few 1e-7 past 1 when the distributions agree)
        const float cstar = fminf(s, 1.f);
        const float d1 = 1.f - cstar;
        const float c_ce = lse[2 * p] - dy[p];
        const float z = zc[p];
        // -(c log sigmoid(z) + (1 - c) log(1 - sigmoid(z))) = softplus(z) - c z
        const float sp = fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
        const float c_bce = sp - cstar * z;
        ce[p] = c_ce;
        l1[p] = d1;
        conf[p] = 1.f / (1.f + __expf(-z));
        bce[p] = c_bce;
        const float om = (mask ? mask[p] : 1.f) * __expf(-(float)(p % gamma) / decay);
        if (om != 0.f) tm.x = om, tm.y = om * c_ce, tm.z = om * d1, tm.w = om * c_bce;
    }
    reinterpret_cast<float4*>(terms)[p] = tm;
}

// one workgroup: loss[4] = (L, L_ce, L_l1, L_conf) from the terms, in a fixed order.
__global__ __launch_bounds__(kReduceThreads) void loss_reduce(int64_t M, const float* __restrict__ terms, float a_ce,
                                                              float a_l1, float a_conf, float* __restrict__ loss) {
    __shared__ float r[kReduceThreads][4];
    const int tid = threadIdx.x;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (int64_t p = tid; p < M; p += kReduceThreads) {
        const float4 t = reinterpret_cast<const float4*>(terms)[p];
        s0 += t.x, s1 += t.y, s2 += t.z, s3 += t.w;
    }
    r[tid][0] = s0, r[tid][1] = s1, r[tid][2] = s2, r[tid][3] = s3;
    __syncthreads();
    for (int n = kReduceThreads / 2; n > 0; n >>= 1) {
        if (tid < n)
#pragma unroll
            for (int q = 0; q < 4; ++q) r[tid][q] += r[tid + n][q];
        __syncthreads();
    }
    if (tid == 0) {
        const float sw = r[0][0];
        const float Lce = sw != 0.f ? r[0][1] / sw : 0.f, Ll1 = sw != 0.f ? r[0][2] / sw : 0.f,
                    Lcf = sw != 0.f ? r[0][3] / sw : 0.f;
        loss[0] = a_ce * Lce + a_l1 * Ll1 + a_conf * Lcf;
        loss[1] = Lce;
        loss[2] = Ll1;
        loss[3] = Lcf;
    }
}

struct LossWs {
    float *stats, *l1p, *dy, *lse, *zc, *terms;
};

LossWs carve_loss(void* ws, int64_t M, int64_t nchunk) {
    char* p = static_cast<char*>(ws);
    auto take = [&](size_t bytes) {
        char* q = p;
        p += (bytes + 255) / 256 * 256;
        return reinterpret_cast<float*>(q);
    };
    LossWs s;
    s.stats = take(sizeof(float) * 4 * (size_t)(nchunk * M));
    s.l1p = take(sizeof(float) * (size_t)(nchunk * M));
    s.dy = take(sizeof(float) * (size_t)M);
    s.lse = take(sizeof(float) * 2 * (size_t)M);
    s.zc = take(sizeof(float) * (size_t)M);
    s.terms = take(sizeof(float) * 4 * (size_t)M);
    return s;
}

}  // namespace

size_t block_loss_workspace(int64_t M, int64_t V) {
    const int64_t nchunk = (V + kChunk - 1) / kChunk;
    auto r = [](size_t b) { return (b + 255) / 256 * 256; };
    return r(16 * (size_t)(nchunk * M)) + r(4 * (size_t)(nchunk * M)) + r(4 * (size_t)M) + r(8 * (size_t)M) +
           r(4 * (size_t)M) + r(16 * (size_t)M);
}

bool block_loss_shape_ok(int64_t r, const void* W1, const void* W2, const void* ws) {
    return r == kRank && (uintptr_t)W1 % 16 == 0 && (uintptr_t)W2 % 16 == 0 && (uintptr_t)ws % 16 == 0;
}

hipError_t block_loss_launch(int64_t N, int64_t gamma, int64_t V, int64_t H, const void* U, const void* t,
                             const void* h, const void* W1, const void* W2, const void* w_conf, float b_conf,
                             const int32_t* xp, const int32_t* y, const float* mask, float decay, float a_ce,
                             float a_l1, float a_conf, float* ce, float* l1, float* conf, float* bce, float* loss,
                             void* ws, hipStream_t stream) {
    const int64_t M = N * gamma;
    const int64_t nchunk = (V + kChunk - 1) / kChunk;
    const LossWs s = carve_loss(ws, M, nchunk);
    const bf16_t* Ub = static_cast<const bf16_t*>(U);
    const bf16_t* Tb = static_cast<const bf16_t*>(t);
    const bf16_t* W1b = static_cast<const bf16_t*>(W1);
    const bf16_t* W2b = static_cast<const bf16_t*>(W2);
    if (M == 0) {  // no positions: the loss terms are zero
        hipLaunchKernelGGL(loss_reduce, dim3(1), dim3(kReduceThreads), 0, stream, M, s.terms, a_ce, a_l1, a_conf,
                           loss);
        return hipGetLastError();
    }
    const bool vec = V % 8 == 0 && (uintptr_t)U % 16 == 0 && (uintptr_t)t % 16 == 0;
    const int64_t total = nchunk * ((M + kBlk - 1) / kBlk);
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const dim3 grid((uint32_t)(total < cus ? total : cus));
    if (vec)
        hipLaunchKernelGGL((loss_stream<1, true>), grid, dim3(kSThreads), 0, stream, M, V, nchunk, Ub, Tb, W1b,
                           W2b, xp, s.stats, s.lse, s.l1p);
    else
        hipLaunchKernelGGL((loss_stream<1, false>), grid, dim3(kSThreads), 0, stream, M, V, nchunk, Ub, Tb,
                           W1b, W2b, xp, s.stats, s.lse, s.l1p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(loss_merge, dim3((uint32_t)M), dim3(256), 0, stream, M, V, H, nchunk, s.stats, Ub,
                       static_cast<const bf16_t*>(h), W1b, W2b, static_cast<const bf16_t*>(w_conf), b_conf, xp, y,
                       s.lse, s.dy, s.zc);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (vec)
        hipLaunchKernelGGL((loss_stream<2, true>), grid, dim3(kSThreads), 0, stream, M, V, nchunk, Ub, Tb, W1b,
                           W2b, xp, s.stats, s.lse, s.l1p);
    else
        hipLaunchKernelGGL((loss_stream<2, false>), grid, dim3(kSThreads), 0, stream, M, V, nchunk, Ub, Tb,
                           W1b, W2b, xp, s.stats, s.lse, s.l1p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(loss_final, dim3((uint32_t)((M + 3) / 4)), dim3(256), 0, stream, M, gamma, V, nchunk,
                       s.l1p, s.dy, s.lse, s.zc, xp, y, mask, decay, ce, l1, conf, bce, s.terms);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(loss_reduce, dim3(1), dim3(kReduceThreads), 0, stream, M, s.terms, a_ce, a_l1, a_conf, loss);
    return hipGetLastError();
}

}  // namespace dspark
