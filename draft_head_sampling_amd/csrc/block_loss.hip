// Teacher-forced block bias with the joint training loss ("基于 DSpark 的投机解码
// 训练框架原理与实现", wangjunjian.com, section 7.2, the joint loss; the
// training loop applies the sequential head with the given previous tokens,
// section 3.2 and paper eq. 5 for the bias).
//
// With the previous tokens given, every position is independent:
//   d[p][v] = U[p][v] + W2[v] . W1[xp[p]]            (draft logits)
// and the loss needs, per position, logsumexp(d), d[y], and
// L1 = 1/2 sum_v |softmax(d)_v - softmax(t)_v|, which needs both row
// normalisers before it can be summed.  Four launches:
//   loss_tiles<1>  a 64-position x 512-row tile of d on the matrix cores
//                  (bf16 in, fp32 accumulate) with the U and t tiles staged
//                  through LDS; per lane an online max/sum of d and t; the
//                  partial (max, sum) pairs of each vocabulary chunk go to
//                  the workspace, and the chunk holding y writes d[y];
//   loss_merge     per position: the chunk partials merged in a fixed order
//                  into logsumexp(d) and logsumexp(t), and the confidence
//                  logit w . [h; W1[xp]] + b;
//   loss_tiles<2>  the same tiles again, summing |p_d - p_t| per chunk;
//   loss_final     per position: L1, CE, c* = 1 - L1, conf, BCE and the
//                  position's weighted terms; then one workgroup sums the
//                  terms over positions in a fixed order.
// Every workspace word is written before it is read, so the workspace needs
// no clearing, and every reduction runs in a fixed order: repeated calls are
// bitwise identical.
#include "block_loss.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRank = 256;          // Markov rank of the matrix-core tiles
constexpr int kRows = 128;          // vocabulary rows per tile (32 per wave)
constexpr int kPos = 64;            // positions per workgroup (two 32-wide MFMA tiles)
constexpr int kTiles = 4;           // tiles per vocabulary chunk
constexpr int kChunk = kRows * kTiles;
constexpr int kERow = kRank + 8;    // LDS row stride of the embeddings (bf16)
constexpr int kTRow = kRows + 8;    // LDS row stride of the U and t tiles (bf16)
constexpr int kReduceThreads = 1024;

__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// (m, s) pairs of an online softmax normaliser: merge b into a.
__device__ __forceinline__ void merge_ms(float& m, float& s, float mb, float sb) {
    const float mm = fmaxf(m, mb);
    if (mm == -INFINITY) return;  // both empty
    s = s * __expf(m - mm) + sb * __expf(mb - mm);
    m = mm;
}

// A 64-position x 128-row tile of X (U or t) as 16-byte pieces, 4 per thread:
// piece c covers position c / 16, rows 8 (c % 16) .. + 7.  Positions past M
// repeat the last one; rows past V read as zero (and are never used).
template <bool VEC>
__device__ __forceinline__ void load_tile(const bf16_t* __restrict__ X, int64_t M, int64_t V, int64_t p0,
                                          int64_t vt, int tid, u32x4_t (&s)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, pl = c / 16, col = (c % 16) * 8;
        const int64_t p = p0 + pl < M ? p0 + pl : M - 1;
        const int64_t v = vt + col;
        const uint16_t* row = reinterpret_cast<const uint16_t*>(X + p * V);
        if (VEC && v + 8 <= V) {
            s[i] = *reinterpret_cast<const u32x4_t*>(row + v);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = v + 2 * j < V ? row[v + 2 * j] : 0u;
                const uint32_t hi = v + 2 * j + 1 < V ? row[v + 2 * j + 1] : 0u;
                w[j] = lo | hi << 16;
            }
            s[i] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
    }
}

// grid (ceil(M / 64), ceil(V / 512)), 256 threads.  PASS 1 writes the
// chunk's (max, sum) of d and t per position to stats [M][chunks][4] and d[y]
// to dy [M]; PASS 2 reads lse [M][2] and writes the chunk's sum of
// |p_d - p_t| to l1p [M][chunks].
template <int PASS, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void loss_tiles(int64_t M, int64_t V, int64_t nchunk, const bf16_t* __restrict__ U,
                                                  const bf16_t* __restrict__ T, const bf16_t* __restrict__ W1,
                                                  const bf16_t* __restrict__ W2, const int32_t* __restrict__ xp,
                                                  const int32_t* __restrict__ y, float* __restrict__ stats,
                                                  float* __restrict__ dy, const float* __restrict__ lse,
                                                  float* __restrict__ l1p) {
    __shared__ __align__(16) uint16_t E_lds[kPos * kERow];
    __shared__ __align__(16) uint16_t U_lds[kPos * kTRow];
    __shared__ __align__(16) uint16_t T_lds[kPos * kTRow];
    __shared__ float red[4][kPos][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, row = lane & 31, half = lane >> 5;
    const int64_t p0 = (int64_t)blockIdx.x * kPos;
    const int64_t chunk = blockIdx.y;

    // embeddings W1[xp] of the 64 positions: 4 threads per position, 128 bytes each
    {
        const int pl = tid >> 2, part = tid & 3;
        const int64_t p = p0 + pl < M ? p0 + pl : M - 1;
        int32_t x = xp[p];
        if (x < 0 || x >= V) x = 0;  // such a position's outputs are NaN; any row will do
        const uint4* src = reinterpret_cast<const uint4*>(W1 + (int64_t)x * kRank + part * 64);
        uint4 e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = src[i];
        uint4* dst = reinterpret_cast<uint4*>(E_lds + pl * kERow + part * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = e[i];
    }
    float md[2], sd[2], mt[2], st[2], l1[2], ld[2], lt[2];
    int32_t yv[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int64_t p = p0 + nt * 32 + row, pc = p < M ? p : M - 1;
        md[nt] = mt[nt] = -INFINITY;
        sd[nt] = st[nt] = l1[nt] = 0.f;
        yv[nt] = y[pc];
        if (PASS == 2) ld[nt] = lse[2 * pc], lt[nt] = lse[2 * pc + 1];
    }
    __syncthreads();

    // In pass 2 the loads of tile i + 1 (W2 fragments, U and t pieces) are
    // issued once tile i's products are done and its U/t pieces are in LDS, so
    // they are in flight during tile i's epilogue.  Pass 1 issues each tile's
    // loads at the tile's start: its epilogue holds more state, and at two
    // waves per SIMD the prefetched registers would spill.
    constexpr bool kPrefetch = PASS == 2;
    // W2 rows of a wave as A fragments: k-step s takes rank elements 16 s + 8 half .. + 7
    auto issue = [&](int64_t vt, uint4(&a)[16], u32x4_t(&us)[4], u32x4_t(&ts)[4]) {
        const int64_t v = vt + wave * 32 + row < V ? vt + wave * 32 + row : V - 1;
        const uint4* src = reinterpret_cast<const uint4*>(W2 + v * kRank + half * 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = src[2 * i];
        load_tile<VEC>(U, M, V, p0, vt, tid, us);
        load_tile<VEC>(T, M, V, p0, vt, tid, ts);
    };
    uint4 a_pf[16];
    u32x4_t us_pf[4], ts_pf[4];
    if (kPrefetch) issue(chunk * kChunk, a_pf, us_pf, ts_pf);  // the grid has no chunk past V
    for (int tile = 0; tile < kTiles; ++tile) {
        const int64_t vt = chunk * kChunk + (int64_t)tile * kRows;
        if (vt >= V) break;  // the same for the whole workgroup
        const int64_t vn = vt + kRows;
        const bool next = tile + 1 < kTiles && vn < V;
        uint4 a_loc[16];
        u32x4_t us_loc[4], ts_loc[4];
        uint4(&a)[16] = kPrefetch ? a_pf : a_loc;
        u32x4_t(&us)[4] = kPrefetch ? us_pf : us_loc;
        u32x4_t(&ts)[4] = kPrefetch ? ts_pf : ts_loc;
        if (!kPrefetch) issue(vt, a, us, ts);
        f32x16_t acc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a[s]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint4 bw = *reinterpret_cast<const uint4*>(E_lds + (nt * 32 + row) * kERow + s * 16 + half * 8);
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bw), acc[nt], 0, 0,
                                                                  0);
            }
        }
        __syncthreads();  // the previous tile's epilogue is done with the staged tiles
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, pl = c / 16, col = (c % 16) * 8;
            *reinterpret_cast<u32x4_t*>(U_lds + pl * kTRow + col) = us[i];
            *reinterpret_cast<u32x4_t*>(T_lds + pl * kTRow + col) = ts[i];
        }
        __syncthreads();
        if (kPrefetch && next) issue(vn, a, us, ts);
        // lane holds rows vt + wave*32 + 8(r/4) + 4 half + r%4 of position nt*32 + row
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int pl = nt * 32 + row;
            // d and t of element r (rows past V: -inf); read again from LDS
            // in each sweep rather than held, which keeps the register count
            // at two waves per SIMD
            auto dval = [&](int r) {
                const int vl = wave * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                return vt + vl < V ? bf(U_lds[pl * kTRow + vl]) + acc[nt][r] : -INFINITY;
            };
            auto tval = [&](int r) {
                const int vl = wave * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                return vt + vl < V ? bf(T_lds[pl * kTRow + vl]) : -INFINITY;
            };
            if (PASS == 1) {
                float mdn = -INFINITY, mtn = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float dr = dval(r);
                    mdn = fmaxf(mdn, dr);
                    mtn = fmaxf(mtn, tval(r));
                    const int64_t v = vt + wave * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                    if (v == yv[nt] && v < V && p0 + pl < M) dy[p0 + pl] = dr;
                }
                if (mdn > -INFINITY) {  // the lane has rows in this tile
                    float s1 = 0.f, s2 = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) s1 += __expf(dval(r) - mdn), s2 += __expf(tval(r) - mtn);
                    merge_ms(md[nt], sd[nt], mdn, s1);
                    merge_ms(mt[nt], st[nt], mtn, s2);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float dr = dval(r);
                    if (dr > -INFINITY) l1[nt] += fabsf(__expf(dr - ld[nt]) - __expf(tval(r) - lt[nt]));
                }
            }
        }
    }

    // the two lanes of a position (half 0 and 1), then the four waves, in order
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int pl = nt * 32 + row;
        if (PASS == 1) {
            const float m2 = __shfl_xor(md[nt], 32), s2 = __shfl_xor(sd[nt], 32);
            const float m3 = __shfl_xor(mt[nt], 32), s3 = __shfl_xor(st[nt], 32);
            if (half == 0) {
                merge_ms(md[nt], sd[nt], m2, s2);
                merge_ms(mt[nt], st[nt], m3, s3);
                red[wave][pl][0] = md[nt], red[wave][pl][1] = sd[nt];
                red[wave][pl][2] = mt[nt], red[wave][pl][3] = st[nt];
            }
        } else {
            const float o = __shfl_xor(l1[nt], 32);
            if (half == 0) red[wave][pl][0] = l1[nt] + o;
        }
    }
    __syncthreads();
    if (tid < kPos && p0 + tid < M) {
        const int64_t p = p0 + tid;
        if (PASS == 1) {
            float m1 = red[0][tid][0], s1 = red[0][tid][1], m2 = red[0][tid][2], s2 = red[0][tid][3];
            for (int w = 1; w < 4; ++w) {
                merge_ms(m1, s1, red[w][tid][0], red[w][tid][1]);
                merge_ms(m2, s2, red[w][tid][2], red[w][tid][3]);
            }
            float4 o;
            o.x = m1, o.y = s1, o.z = m2, o.w = s2;
            reinterpret_cast<float4*>(stats)[p * nchunk + chunk] = o;
        } else {
            l1p[p * nchunk + chunk] = ((red[0][tid][0] + red[1][tid][0]) + red[2][tid][0]) + red[3][tid][0];
        }
    }
}

// grid M, 256 threads: lse [M][2] = (logsumexp d, logsumexp t) from the chunk
// partials, and the confidence logit z [M] = w . [h; W1[xp]] + b.
__global__ __launch_bounds__(256) void loss_merge(int64_t M, int64_t V, int64_t H, int64_t nchunk,
                                                  const float* __restrict__ stats, const bf16_t* __restrict__ h,
                                                  const bf16_t* __restrict__ W1, const bf16_t* __restrict__ w,
                                                  float b_conf, const int32_t* __restrict__ xp,
                                                  float* __restrict__ lse, float* __restrict__ zc) {
    __shared__ float rm[256][4];
    __shared__ float rz[4];
    const int64_t p = blockIdx.x;
    const int tid = threadIdx.x;
    float m1 = -INFINITY, s1 = 0.f, m2 = -INFINITY, s2 = 0.f;
    for (int64_t c = tid; c < nchunk; c += 256) {
        const float4 o = reinterpret_cast<const float4*>(stats)[p * nchunk + c];
        merge_ms(m1, s1, o.x, o.y);
        merge_ms(m2, s2, o.z, o.w);
    }
    rm[tid][0] = m1, rm[tid][1] = s1, rm[tid][2] = m2, rm[tid][3] = s2;
    int32_t x = xp[p];
    if (x < 0 || x >= V) x = 0;
    float z = 0.f;
    for (int64_t i = tid; i < H + kRank; i += 256)
        z += load_elem(w, i) * (i < H ? load_elem(h, p * H + i) : load_elem(W1, (int64_t)x * kRank + (i - H)));
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    if ((tid & 63) == 0) rz[tid >> 6] = z;
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
        const float d1 = 0.5f * s;
        const float c_ce = lse[2 * p] - dy[p];
        const float cstar = 1.f - d1;
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
    const dim3 grid((uint32_t)((M + kPos - 1) / kPos), (uint32_t)nchunk);
    if (vec)
        hipLaunchKernelGGL((loss_tiles<1, true>), grid, dim3(256), 0, stream, M, V, nchunk, Ub, Tb, W1b, W2b, xp, y,
                           s.stats, s.dy, s.lse, s.l1p);
    else
        hipLaunchKernelGGL((loss_tiles<1, false>), grid, dim3(256), 0, stream, M, V, nchunk, Ub, Tb, W1b, W2b, xp, y,
                           s.stats, s.dy, s.lse, s.l1p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(loss_merge, dim3((uint32_t)M), dim3(256), 0, stream, M, V, H, nchunk, s.stats,
                       static_cast<const bf16_t*>(h), W1b, static_cast<const bf16_t*>(w_conf), b_conf, xp, s.lse,
                       s.zc);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (vec)
        hipLaunchKernelGGL((loss_tiles<2, true>), grid, dim3(256), 0, stream, M, V, nchunk, Ub, Tb, W1b, W2b, xp, y,
                           s.stats, s.dy, s.lse, s.l1p);
    else
        hipLaunchKernelGGL((loss_tiles<2, false>), grid, dim3(256), 0, stream, M, V, nchunk, Ub, Tb, W1b, W2b, xp, y,
                           s.stats, s.dy, s.lse, s.l1p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(loss_final, dim3((uint32_t)((M + 3) / 4)), dim3(256), 0, stream, M, gamma, V, nchunk,
                       s.l1p, s.dy, s.lse, s.zc, xp, y, mask, decay, ce, l1, conf, bce, s.terms);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(loss_reduce, dim3(1), dim3(kReduceThreads), 0, stream, M, s.terms, a_ce, a_l1, a_conf, loss);
    return hipGetLastError();
}

}  // namespace dspark
