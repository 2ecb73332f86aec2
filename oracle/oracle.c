/*
 * CPU oracle for the DSpark draft-head hot path.  TEST INFRASTRUCTURE ONLY:
 * nothing but the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load or call this library.  The product path never routes here.
 *
 * Plain, slow, single-threaded definitions, accumulated in double.  Inputs in
 * bfloat16 are widened exactly (a bfloat16 is the upper half of a binary32).
 * This file shares no code with the HIP path.
 *
 * Sources (the pages describing the method):
 *   [W]  "基于 DSpark 的投机解码训练框架原理与实现（论文+代码对照）",
 *        wangjunjian.com -- section 3.2 (semi-autoregressive generation:
 *        p_k(v) = softmax(U_k(v) + B_k(x_0, x_<k, v)); the vanilla Markov head,
 *        paper eq. 5, B(x_{k-1}, .) = W2 . W1[x_{k-1}], rank r; the block
 *        sampling loop of sample_block_tokens), section 3.3 (confidence head
 *        fed with h_k and the previous token's Markov embedding W1[x_{k-1}];
 *        analytic accept rate, paper eq. 8, c* = 1 - 1/2 ||p_d - p_t||_1;
 *        Algorithm 1, the hardware-aware prefix scheduler), section 8.2
 *        (rejection-sampling verification, accept with min(1, p_t/p_d)).
 *   [D]  dpshk.com article on the Qwen3.8-27B-DSpark confidence head,
 *        section 2 (AcceptRatePredictor is one nn.Linear(input_dim, 1) that
 *        returns a logit) and section 3 (config.json: confidence head fed with
 *        the Markov feature, markov_rank 256, hidden 5120, block 7).
 *
 * Readings where the pages leave a step open (each also listed in the
 * design notes):
 *   - sample(): greedy = argmax of the step logits; Gumbel-max = argmax of
 *     logits + supplied Gumbel noise (temperature 1).  The argmax decision is
 *     taken in binary32, the precision of the GPU kernels, on the fp64 score
 *     rounded once to binary32; exact ties go to the lowest token id.
 *   - the confidence head's sigmoid is applied to the linear head's logit;
 *     its input is [h_k ; W1[x_{k-1}]], x_0 = the anchor.
 *   - survival a_k = prod_{i<=k} c_i.
 *   - scheduler: survivals are binary32 sequential products; pairs are sorted
 *     by (survival desc, request asc, position asc); the empty selection has
 *     tau = B (one bonus token per request) and Btok = B; a pair is accepted
 *     iff Theta = (tau + a) * SPS(Btok + 1) > Theta_best strictly; the first
 *     pair that fails, or that would need a batch beyond the table, stops
 *     the scan.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact value of element i of a float32 or bfloat16 buffer. */
static double val(const void* p, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Block sampler with the vanilla Markov head and the confidence head.
 *
 * For each request b, x = x0[b], A = 1.  For k = 1..gamma ([W] 3.2, the
 * sampling loop; eq. 5; [W] 3.3 and [D] 2 for the confidence head):
 *   e[j]      = W1[x, j]                               (previous-token embedding)
 *   bias[v]   = sum_j W2[v, j] * e[j]                  (eq. 5)
 *   logit[v]  = U[b, k, v] + bias[v]                   (step logits)
 *   score[v]  = logit[v] + G[b, k, v]   (G absent -> 0; Gumbel-max draw)
 *   tokens    = lowest v maximising binary32(score[v])
 *   margin    = largest minus second-largest score (fp64, over distinct v)
 *   c_k       = sigmoid(sum_i w[i] h[b,k,i] + sum_j w[H+j] e[j] + b_conf)
 *   A_k       = A_{k-1} * c_k
 *   x         = force[b, k] if given (>= 0) else the sampled token
 *
 * Shapes: U, G [B][gamma][V]; h [B][gamma][H]; W1, W2 [V][r]; w [H + r].
 * Outputs tokens, conf, survival, margin [B][gamma]; logits and bias
 * [B][gamma][V] may be NULL.  Returns 0, or -1 on a token id outside [0, V).
 *
 * Gated Markov head ([W] 3.2, the second of the three sequential heads), when
 * Wg [r][H + r] is given: the embedding is gated by the hidden state and
 * itself before the projection,
 *   g[j]      = sigmoid(sum_i Wg[j, i] h[b,k,i] + sum_i Wg[j, H+i] e[i])
 *   bias[v]   = sum_j W2[v, j] * (g[j] * e[j])
 * (the pages give B = sigma(Wg [h_k; W1[x_{k-1}]]) (x) W1[x_{k-1}] and leave the
 * map back to the vocabulary open; the plainest reading is the same W2 as
 * the vanilla head).  The confidence head still sees e itself.
 *
 * RNN head ([W] 3.2, paper eq. 6), when Wrg and Wrc [r][2r + H] are given: a
 * recurrent state s (s_0 = 0) replaces the embedding in the bias,
 *   z         = [s_{k-1} ; e ; h[b,k,:]]
 *   u[j]      = sigmoid(sum_i Wrg[j, i] z[i])
 *   s_k[j]    = u[j] s_{k-1}[j] + (1 - u[j]) tanh(sum_i Wrc[j, i] z[i])
 *   bias[v]   = sum_j W2[v, j] s_k[j]
 * (the pages' "(1-sigma)(Wg z)" is read as 1 - sigmoid(Wg z), the GRU-style
 * update; the map back to the vocabulary is read as W2).  The confidence head
 * still sees e.
 */
int oracle_head_sample(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int dtype, const void* U,
                       const void* h, const void* W1, const void* W2, const void* w, double b_conf,
                       const int32_t* x0, const float* gumbel, const int32_t* force, int32_t* tokens,
                       double* conf, double* survival, double* margin, double* logits, double* bias,
                       const void* Wg, const void* Wrg, const void* Wrc) {
    const size_t rn = (size_t)(r > 0 ? r : 1);
    double* e = (double*)malloc(sizeof(double) * rn);
    double* eb = (double*)malloc(sizeof(double) * rn); /* what the bias sees */
    double* st = (double*)malloc(sizeof(double) * rn); /* the RNN state */
    if (!e || !eb || !st) {
        free(e);
        free(eb);
        free(st);
        return -2;
    }
    const int64_t Z = 2 * r + H; /* RNN input width */
    for (int64_t b = 0; b < B; ++b) {
        int64_t x = x0[b];
        double A = 1.0;
        for (int64_t j = 0; j < r; ++j) st[j] = 0.0;
        for (int64_t k = 0; k < gamma; ++k) {
            if (x < 0 || x >= V) {
                free(e);
                free(eb);
                free(st);
                return -1;
            }
            for (int64_t j = 0; j < r; ++j) e[j] = val(W1, dtype, x * r + j);
            for (int64_t j = 0; j < r; ++j) {
                eb[j] = e[j];
                if (Wg) {
                    double z = 0.0;
                    for (int64_t i = 0; i < H; ++i)
                        z += val(Wg, dtype, j * (H + r) + i) * val(h, dtype, (b * gamma + k) * H + i);
                    for (int64_t i = 0; i < r; ++i) z += val(Wg, dtype, j * (H + r) + H + i) * e[i];
                    eb[j] = e[j] / (1.0 + exp(-z));
                }
            }
            if (Wrg && Wrc) {
                const int64_t hz = (b * gamma + k) * H;
                for (int64_t j = 0; j < r; ++j) {
                    double zg = 0.0, zc = 0.0;
                    for (int64_t i = 0; i < r; ++i) {
                        zg += val(Wrg, dtype, j * Z + i) * st[i];
                        zc += val(Wrc, dtype, j * Z + i) * st[i];
                    }
                    for (int64_t i = 0; i < r; ++i) {
                        zg += val(Wrg, dtype, j * Z + r + i) * e[i];
                        zc += val(Wrc, dtype, j * Z + r + i) * e[i];
                    }
                    for (int64_t i = 0; i < H; ++i) {
                        zg += val(Wrg, dtype, j * Z + 2 * r + i) * val(h, dtype, hz + i);
                        zc += val(Wrc, dtype, j * Z + 2 * r + i) * val(h, dtype, hz + i);
                    }
                    const double u = 1.0 / (1.0 + exp(-zg));
                    eb[j] = u * st[j] + (1.0 - u) * tanh(zc);
                }
                for (int64_t j = 0; j < r; ++j) st[j] = eb[j];
            }

            const int64_t row = (b * gamma + k) * V;
            int64_t best = -1;
            float best32 = 0.0f;
            double top1 = -INFINITY, top2 = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                double s = 0.0;
                for (int64_t j = 0; j < r; ++j) s += val(W2, dtype, v * r + j) * eb[j];
                double lg = val(U, dtype, row + v) + s;
                double sc = lg + (gumbel ? (double)gumbel[row + v] : 0.0);
                if (bias) bias[row + v] = s;
                if (logits) logits[row + v] = lg;
                float sc32 = (float)sc;
                if (best < 0 || sc32 > best32) {
                    best = v;
                    best32 = sc32;
                }
                if (sc > top1) {
                    top2 = top1;
                    top1 = sc;
                } else if (sc > top2) {
                    top2 = sc;
                }
            }
            tokens[b * gamma + k] = (int32_t)best;
            if (margin) margin[b * gamma + k] = top1 - top2;

            double z = b_conf;
            for (int64_t i = 0; i < H; ++i) z += val(w, dtype, i) * val(h, dtype, (b * gamma + k) * H + i);
            for (int64_t j = 0; j < r; ++j) z += val(w, dtype, H + j) * e[j];
            double c = 1.0 / (1.0 + exp(-z));
            A *= c;
            conf[b * gamma + k] = c;
            survival[b * gamma + k] = A;

            x = (force && force[b * gamma + k] >= 0) ? force[b * gamma + k] : best;
        }
    }
    free(e);
    free(eb);
    free(st);
    return 0;
}

/*
 * Analytic accept rate, [W] 3.3, paper eq. 8: per row n
 *   p = softmax(d_n), q = softmax(t_n)
 *   cstar[n] = 1 - 1/2 sum_v |p_v - q_v|
 * and, as a second route to the same number, summin[n] = sum_v min(p_v, q_v)
 * (may be NULL).  Rows are ld elements apart.
 */
int oracle_accept_rate(int64_t N, int64_t V, int dtype, const void* d, int64_t ld_d, const void* t,
                       int64_t ld_t, double* cstar, double* summin) {
    for (int64_t n = 0; n < N; ++n) {
        const int64_t od = n * ld_d, ot = n * ld_t;
        double md = -INFINITY, mt = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            double a = val(d, dtype, od + v), b = val(t, dtype, ot + v);
            if (a > md) md = a;
            if (b > mt) mt = b;
        }
        double sd = 0.0, st = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            sd += exp(val(d, dtype, od + v) - md);
            st += exp(val(t, dtype, ot + v) - mt);
        }
        double l1 = 0.0, mn = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double p = exp(val(d, dtype, od + v) - md) / sd;
            double q = exp(val(t, dtype, ot + v) - mt) / st;
            l1 += fabs(p - q);
            mn += p < q ? p : q;
        }
        cstar[n] = 1.0 - 0.5 * l1;
        if (summin) summin[n] = mn;
    }
    return 0;
}

/* Sort order of Algorithm 1: survival descending, then request, then
 * position ascending (a total order on distinct pairs). */
static const float* g_surv;
static int cmp_pairs(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    float sa = g_surv[a], sb = g_surv[b];
    if (sa > sb) return -1;
    if (sa < sb) return 1;
    return (a > b) - (a < b); /* pair id r*gamma + j orders by (r, j) */
}

/*
 * Hardware-aware prefix scheduler, [W] 3.3, Algorithm 1 (flowchart):
 *   a[r][j]  = c[r][0] * ... * c[r][j]         (binary32, left to right)
 *   sort all (r, j) by a descending
 *   tau = B, Btok = B, Theta_best = B * SPS(B)
 *   for each pair in order:
 *       stop if Btok + 1 > n_sps
 *       Theta = (tau + a) * SPS(Btok + 1)
 *       if Theta > Theta_best: accept, tau += a, Btok += 1,
 *                              l[r] = j + 1, Theta_best = Theta
 *       else stop
 * sps[n-1] = SPS(n).  conf values are in [0, 1].
 * Outputs: prefix_len [B]; survival [B][gamma] and order [B*gamma] (pair ids
 * r*gamma + j in sorted order) may be NULL; theta [1] = Theta_best;
 * n_selected [1] = number of accepted pairs.  Returns 0, -1 if n_sps < B.
 */
int oracle_prefix_schedule(int64_t B, int64_t gamma, const float* conf, const double* sps, int64_t n_sps,
                           int32_t* prefix_len, float* survival, int32_t* order, double* theta,
                           int64_t* n_selected) {
    if (B < 1 || n_sps < B) return -1;
    const int64_t n = B * gamma;
    float* a = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    int32_t* ord = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!a || !ord) {
        free(a);
        free(ord);
        return -2;
    }
    for (int64_t r = 0; r < B; ++r) {
        float p = 1.0f;
        for (int64_t j = 0; j < gamma; ++j) {
            p = p * conf[r * gamma + j];
            a[r * gamma + j] = p;
        }
    }
    for (int64_t i = 0; i < n; ++i) ord[i] = (int32_t)i;
    g_surv = a;
    qsort(ord, (size_t)n, sizeof(int32_t), cmp_pairs);

    for (int64_t r = 0; r < B; ++r) prefix_len[r] = 0;
    double tau = (double)B;
    int64_t btok = B;
    double best = tau * sps[btok - 1];
    int64_t sel = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (btok + 1 > n_sps) break;
        double ai = (double)a[ord[i]];
        double th = (tau + ai) * sps[btok];
        if (!(th > best)) break;
        tau += ai;
        btok += 1;
        best = th;
        prefix_len[ord[i] / gamma] = (int32_t)(ord[i] % gamma + 1);
        ++sel;
    }
    if (survival) memcpy(survival, a, sizeof(float) * (size_t)n);
    if (order) memcpy(order, ord, sizeof(int32_t) * (size_t)n);
    if (theta) *theta = best;
    if (n_selected) *n_selected = sel;
    free(a);
    free(ord);
    return 0;
}

/*
 * Rejection-sampling verification of one draft block per request ([W] 8.2:
 * accept a drafted token with probability min(1, p_target / p_draft); on a
 * rejection drop it and every later one and sample the next token from the
 * residual max(0, p_target - p_draft); [W] 2.1: the target then adds one
 * bonus token after an accepted prefix).
 *
 * Layouts: d [B][gamma][V] draft logits, t [B][gamma + 1][V] target logits,
 * x [B][gamma] drafted tokens, n_draft [B] drafted positions to verify (NULL:
 * gamma; values outside [0, gamma] are clamped), u [B][gamma] uniforms in
 * [0, 1), G [B][V] Gumbel noise for the one sample each request draws.
 *
 * For request b with n drafted tokens, and k = 1..n in order:
 *   p_d = softmax(d[b,k,:]), p_t = softmax(t[b,k,:]);
 *   x_k is accepted iff u[b,k] * p_d(x_k) < p_t(x_k), i.e. u < min(1, p_t/p_d)
 *   for p_d(x_k) > 0 (a token outside [0, V) is rejected);
 *   the first rejection at k ends the walk: the emitted token is a sample
 *   from the residual at position k,
 *       argmax over v with p_t(v) > p_d(v) of  log(p_t(v) - p_d(v)) + G[b,v]
 *   (Gumbel-max over the normalised residual; an empty residual falls back
 *   to p_t itself).
 * If all n are accepted the emitted token is the bonus sample from p_t at
 * position n + 1: argmax of t[b,n+1,v] + G[b,v].  The argmax is decided in
 * binary32 on each fp64 score rounded once; ties go to the lowest id.
 *
 * Outputs: n_acc [B], next_tok [B], and optionally accept_prob [B][gamma]
 * (min(1, p_t(x_k)/p_d(x_k)) for every drafted k <= n, also past the first
 * rejection; 0 for an invalid token, NaN past n), margin [B] (top1 - top2 of the emitted sample's binary32 scores),
 * sample_pos [B] (0-based position of the sample) and residual [B] (1 when
 * the sample came from a residual).
 */
static double lse_row(const void* p, int dtype, int64_t off, int64_t V) {
    double m = -INFINITY, s = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double a = val(p, dtype, off + v);
        if (a > m) m = a;
    }
    for (int64_t v = 0; v < V; ++v) s += exp(val(p, dtype, off + v) - m);
    return m + log(s);
}

int oracle_verify(int64_t B, int64_t gamma, int64_t V, int dtype, const void* d, const void* t, const int32_t* x,
                  const int32_t* n_draft, const float* u, const float* G, int32_t* n_acc, int32_t* next_tok,
                  double* accept_prob, double* margin, int32_t* sample_pos, int32_t* residual) {
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = n_draft ? n_draft[b] : gamma;
        if (n < 0) n = 0;
        if (n > gamma) n = gamma;
        if (accept_prob)
            for (int64_t k = 0; k < gamma; ++k) accept_prob[b * gamma + k] = NAN;
        int64_t k = 0, pos = n;
        int res = 0;
        double Ld = 0.0, Lt = 0.0;
        for (; k < n; ++k) {
            const int64_t od = (b * gamma + k) * V, ot = (b * (gamma + 1) + k) * V;
            const double ld = lse_row(d, dtype, od, V), lt = lse_row(t, dtype, ot, V);
            const int32_t xk = x[b * gamma + k];
            int ok = 0;
            double a = 0.0;
            if (xk >= 0 && xk < V) {
                const double pd = exp(val(d, dtype, od + xk) - ld), pt = exp(val(t, dtype, ot + xk) - lt);
                a = pd > 0.0 ? (pt / pd < 1.0 ? pt / pd : 1.0) : (pt > 0.0 ? 1.0 : 0.0);
                ok = (double)u[b * gamma + k] * pd < pt;
            }
            if (accept_prob) accept_prob[b * gamma + k] = a;
            if (!ok) {
                pos = k, res = 1, Ld = ld, Lt = lt;
                break;
            }
        }
        n_acc[b] = (int32_t)k;
        /* the probabilities of the drafted tokens past a rejection are reported
         * too (they take no part in the decisions) */
        if (accept_prob)
            for (int64_t j = k + 1; j < n; ++j) {
                const int64_t od = (b * gamma + j) * V, ot = (b * (gamma + 1) + j) * V;
                const int32_t xj = x[b * gamma + j];
                double a = 0.0;
                if (xj >= 0 && xj < V) {
                    const double pd = exp(val(d, dtype, od + xj) - lse_row(d, dtype, od, V));
                    const double pt = exp(val(t, dtype, ot + xj) - lse_row(t, dtype, ot, V));
                    a = pd > 0.0 ? (pt / pd < 1.0 ? pt / pd : 1.0) : (pt > 0.0 ? 1.0 : 0.0);
                }
                accept_prob[b * gamma + j] = a;
            }
        /* the sample: residual at the rejected position, else the bonus */
        const int64_t ot = (b * (gamma + 1) + pos) * V, od = (b * gamma + pos) * V;
        int have = 0;
        float best = 0.f, second = -INFINITY;
        int32_t tok = -1;
        for (int pass = 0; pass < 2 && !have; ++pass) {
            /* pass 0: the residual (only after a rejection); pass 1: p_t */
            if (pass == 0 && !res) continue;
            best = -INFINITY, second = -INFINITY, tok = -1;
            for (int64_t v = 0; v < V; ++v) {
                double sc;
                if (pass == 0) {
                    const double r = exp(val(t, dtype, ot + v) - Lt) - exp(val(d, dtype, od + v) - Ld);
                    if (!(r > 0.0)) continue;
                    sc = log(r) + (double)G[b * V + v];
                } else {
                    sc = val(t, dtype, ot + v) + (double)G[b * V + v];
                }
                const float f = (float)sc;
                if (tok < 0 || f > best) {
                    if (tok >= 0) second = best;
                    best = f, tok = (int32_t)v;
                } else if (f > second) {
                    second = f;
                }
                have = 1;
            }
            if (pass == 0 && !have) res = 0; /* empty residual: sample p_t at this position */
        }
        next_tok[b] = tok;
        if (margin) margin[b] = (double)best - (double)second;
        if (sample_pos) sample_pos[b] = (int32_t)pos;
        if (residual) residual[b] = res;
    }
    return 0;
}

/*
 * Teacher-forced block bias with the joint loss ([W] section 7.2, the joint
 * loss of the training loop; the training loop's apply_block_logits step
 * applies the sequential head with given previous tokens).  Positions are
 * [N][gamma]; for each position (n, k), k = 0..gamma-1, with x = xp[n][k]
 * (the given previous token) and y = y[n][k] (the target id):
 *   e[j]     = W1[x, j]
 *   d[v]     = U[n,k,v] + sum_j W2[v, j] e[j]          (draft logits, eq. 5)
 *   ce       = logsumexp(d) - d[y]                     (cross-entropy)
 *   l1       = 1/2 sum_v |softmax(d)_v - softmax(t_nk)_v|
 *   cstar    = 1 - l1                                  (eq. 8)
 *   conf     = sigmoid(sum_i w[i] h[n,k,i] + sum_j w[H+j] e[j] + b_conf)
 *   bce      = -(cstar log(conf) + (1 - cstar) log(1 - conf))
 *   omega    = mask[n][k] * exp(-k / decay)            (position weight,
 *              exp(-(k-1)/gamma_decay) for 1-based k)
 * and the loss is a_ce L_ce + a_l1 L_l1 + a_conf L_conf with each term the
 * omega-weighted mean over the positions that count,
 *   L_x = sum omega x / sum omega        (0 when sum omega = 0).
 * Readings: the pages name the three terms, their weights and the decay but
 * not the reduction over positions; the weighted mean is the plainest one.
 * A position counts when its mask is non-zero and x and y lie in [0, V); a
 * position whose x or y is out of range gets NaN in every per-position
 * output.  mask may be NULL (all ones).
 * Outputs: ce, l1, conf, bce [N][gamma]; loss[4] = (L, L_ce, L_l1, L_conf).
 */
int oracle_block_loss(int64_t N, int64_t gamma, int64_t V, int64_t H, int64_t r, int dtype, const void* U,
                      const void* t, const void* h, const void* W1, const void* W2, const void* w, double b_conf,
                      const int32_t* xp, const int32_t* y, const float* mask, double decay, double a_ce,
                      double a_l1, double a_conf, double* ce, double* l1, double* conf, double* bce, double* loss) {
    double* d = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
    if (!d) return -2;
    double sw = 0.0, s_ce = 0.0, s_l1 = 0.0, s_bce = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < gamma; ++k) {
            const int64_t pos = n * gamma + k;
            const int32_t x = xp[pos], yy = y[pos];
            if (x < 0 || x >= V || yy < 0 || yy >= V) {
                ce[pos] = l1[pos] = conf[pos] = bce[pos] = NAN;
                continue;
            }
            for (int64_t v = 0; v < V; ++v) {
                double b = 0.0;
                for (int64_t j = 0; j < r; ++j) b += val(W2, dtype, v * r + j) * val(W1, dtype, (int64_t)x * r + j);
                d[v] = val(U, dtype, pos * V + v) + b;
            }
            double md = -INFINITY, mt = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                if (d[v] > md) md = d[v];
                const double tv = val(t, dtype, pos * V + v);
                if (tv > mt) mt = tv;
            }
            double sd = 0.0, st = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                sd += exp(d[v] - md);
                st += exp(val(t, dtype, pos * V + v) - mt);
            }
            double dist = 0.0;
            for (int64_t v = 0; v < V; ++v)
                dist += fabs(exp(d[v] - md) / sd - exp(val(t, dtype, pos * V + v) - mt) / st);
            const double c_ce = md + log(sd) - d[yy];
            const double c_l1 = 0.5 * dist;
            const double cstar = 1.0 - c_l1;
            double z = b_conf;
            for (int64_t i = 0; i < H; ++i) z += val(w, dtype, i) * val(h, dtype, pos * H + i);
            for (int64_t j = 0; j < r; ++j) z += val(w, dtype, H + j) * val(W1, dtype, (int64_t)x * r + j);
            const double c = 1.0 / (1.0 + exp(-z));
            const double c_bce = -(cstar * log(c) + (1.0 - cstar) * log(1.0 - c));
            ce[pos] = c_ce;
            l1[pos] = c_l1;
            conf[pos] = c;
            bce[pos] = c_bce;
            const double om = (mask ? (double)mask[pos] : 1.0) * exp(-(double)k / decay);
            if (om != 0.0) {
                sw += om;
                s_ce += om * c_ce;
                s_l1 += om * c_l1;
                s_bce += om * c_bce;
            }
        }
    }
    free(d);
    const double Lce = sw != 0.0 ? s_ce / sw : 0.0, Ll1 = sw != 0.0 ? s_l1 / sw : 0.0,
                 Lcf = sw != 0.0 ? s_bce / sw : 0.0;
    loss[0] = a_ce * Lce + a_l1 * Ll1 + a_conf * Lcf;
    loss[1] = Lce;
    loss[2] = Ll1;
    loss[3] = Lcf;
    return 0;
}
