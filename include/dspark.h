/*
 * dspark.h -- C ABI of the MI355X (gfx950) draft-head hot path of DSpark's
 * semi-autoregressive drafter: the Markov-head block sampler with its
 * confidence head, the analytic accept rate, and the hardware-aware prefix
 * scheduler.
 *
 * Sources:
 *   [W] "基于 DSpark 的投机解码训练框架原理与实现（论文+代码对照）" (wangjunjian.com),
 *       sections 3.2, 3.3 and 8.2.
 *   [D] dpshk.com article on the Qwen3.8-27B-DSpark confidence head
 *       (AcceptRatePredictor), sections 2 and 3.
 *
 * Conventions shared by every entry point:
 *   - Array pointers are DEVICE pointers on the current HIP device, owned by
 *     the caller.  Scalars are host values.  The library keeps no pointer
 *     after a call returns, allocates no memory and holds no mutable global
 *     state apart from the wait limit (dspark_set_wait_limit); concurrent
 *     calls are safe when they use distinct workspaces.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) without host synchronisation.  Outputs are valid once the
 *     stream has reached the point of the call.
 *   - Workspace: device scratch owned by the caller.  dspark_*_workspace_size
 *     returns the bytes an entry point needs for given shapes (0 means the
 *     workspace argument may be NULL).  A workspace must be at least that
 *     large and 256-byte aligned; workspace_bytes is its size.  It must be
 *     zero-filled before its first use; every call that completes without a
 *     give-up (below) leaves it zero-filled again, except for the path-flags
 *     word, so one workspace serves any number of calls in stream order.
 *     Calls that may overlap in time must not share a workspace.
 *   - Persistent kernels and give-ups.  The B = 1 and batched (16 <= B <= 64,
 *     bf16, r = 256) samplers, the accept rate on 16-byte aligned rows and
 *     the draw of dspark_verify let workgroups wait for one another through
 *     the workspace.  The first three size their grids so that every
 *     workgroup is resident at once on a GPU that runs nothing else (at most
 *     one workgroup per compute unit, or the occupancy limit); they do not
 *     use cooperative launch.  Every such wait is bounded (about 2^21 to
 *     2^22 polls by default, see dspark_set_wait_limit).  When a wait runs
 *     out -- typically because other work held compute units and a
 *     workgroup could not start -- the kernel still finishes, the affected
 *     outputs are token -1 / NaN (outputs of such a call are unspecified),
 *     and word 1 of the workspace header is set.  Read it with
 *     dspark_workspace_status.  Recovery: zero-fill the whole workspace
 *     before its next use (words of the lost workgroups may still be set).
 *   - Errors: every argument check runs on the host before anything is
 *     enqueued; on failure a non-zero status is returned and nothing is
 *     enqueued.  A failed launch returns DSPARK_ERR_HIP.  No C++ exception
 *     crosses this interface.
 *   - Empty sampler and accept-rate problems (B == 0, gamma == 0, N == 0)
 *     are valid and enqueue nothing.  The scheduler needs B >= 1 and always
 *     writes its outputs (gamma == 0 selects nothing).
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_OK = 0,
    DSPARK_ERR_NULL_ARG = 1,  /* a required pointer is NULL */
    DSPARK_ERR_BAD_SHAPE = 2, /* a size is negative, zero where it may not be, or too large */
    DSPARK_ERR_BAD_DTYPE = 3, /* dtype is not one of dspark_dtype_t */
    DSPARK_ERR_WORKSPACE = 4, /* workspace too small or misaligned */
    DSPARK_ERR_HIP = 5        /* a HIP call or kernel launch failed */
} dspark_status_t;

typedef enum {
    DSPARK_F32 = 0, /* IEEE binary32 */
    DSPARK_BF16 = 1 /* bfloat16: the upper 16 bits of a binary32 */
} dspark_dtype_t;

/*
 * dspark_head_sample -- sequential Markov-head block sampler, confidence head
 * and survival products for one draft block of `gamma` positions for each of
 * `B` requests ([W] 3.2: p_k(v) proportional to exp(U_k(v) + B_k(x_{k-1}, v)),
 * the vanilla Markov head B(x_{k-1}, .) = W2 . W1[x_{k-1}] of paper eq. 5,
 * and the block sampling loop in which each sampled token feeds the next
 * step; [W] 3.3 and [D] 2 for the confidence head; [W] 3.3 Algorithm 1 for
 * the survival products).
 *
 * For every request b, with x_0 = x0[b], and k = 1..gamma:
 *   e          = W1[x_{k-1}, :]                          (row gather)
 *   bias[v]    = sum_j W2[v, j] * e[j]                   (fp32 accumulation)
 *   logit[v]   = U[b, k, v] + bias[v]
 *   tokens[b,k]= argmax_v (logit[v] + G[b, k, v])        (G = 0 if gumbel == NULL;
 *                                                         exact ties -> lowest v)
 *   conf[b,k]  = sigmoid(sum_i w_conf[i] h[b,k,i] + sum_j w_conf[H+j] e[j] + b_conf)
 *   survival   = conf[b,1] * ... * conf[b,k]
 *   x_k        = force[b,k] if force != NULL and force[b,k] >= 0, else tokens[b,k]
 * All arithmetic is binary32; bf16 inputs are widened exactly.
 *
 * Arguments (row-major, innermost dimension last):
 *   B, gamma, V, H, r  requests, block width, vocabulary, hidden size, Markov
 *                      rank.  0 <= B <= 524280; gamma >= 0; 1 <= V < 2^31;
 *                      H >= 0; 1 <= r <= 1024.
 *   dtype              dtype of U, h, W1, W2 and w_conf (all the same).
 *   U      [B][gamma][V]  base logits of the parallel backbone.
 *   h      [B][gamma][H]  backbone hidden states (may be NULL if H == 0).
 *   W1     [V][r]         Markov embedding, gathered by the previous token.
 *   W2     [V][r]         Markov output factor.
 *   w_conf [H + r]        confidence weights, ordered [hidden part; Markov part].
 *   b_conf                confidence bias.
 *   x0     [B] int32      anchor tokens.
 *   gumbel [B][gamma][V] fp32 Gumbel noise for Gumbel-max sampling, or NULL
 *                         for greedy argmax.
 *   force  [B][gamma] int32 teacher-forced tokens (-1 = use the sample), or NULL.
 *   tokens [B][gamma] int32      out: sampled tokens.
 *   conf, survival [B][gamma] fp32 out.
 *   logits_out [B][gamma][V] fp32 out, optional (NULL = not written): U + bias.
 *   bias_out   [B][gamma][V] fp32 out, optional (NULL = not written).
 * A token id outside [0, V) in x0 or force makes that request's tokens -1 and
 * its conf and survival NaN from that step on; other requests are unaffected.
 * Scores compare as binary32 values (-0 equals +0, infinities allowed); with a
 * NaN score anywhere in a step the token of that step is unspecified.
 */
dspark_status_t dspark_head_sample(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype,
                                   const void* U, const void* h, const void* W1, const void* W2,
                                   const void* w_conf, float b_conf, const int32_t* x0, const float* gumbel,
                                   const int32_t* force, int32_t* tokens, float* conf, float* survival,
                                   float* logits_out, float* bias_out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * dspark_w2_bound -- weights-only bound for the single-request sampler's
 * candidate screen ([W] 3.2, the sampling loop: a step's winner is proved
 * from U and a bound on |W2[v] . e|, and that bound needs the largest row
 * norm of W2).  Computed once per weight load; dspark_head_sample_w2bound
 * then skips the pass over W2 that each call otherwise makes for it.
 *   V >= 1, r == 256, dtype DSPARK_BF16, W2 [V][r] 16-byte aligned (the
 *   shapes the screen runs on); otherwise DSPARK_ERR_BAD_SHAPE / _BAD_DTYPE.
 *   bound [DSPARK_W2_BOUND_WORDS] uint32, DEVICE memory, out:
 *     bound[0]  the largest squared row norm (binary32 bits, rounded as the
 *               screen rounds it)
 *     bound[1]  the same over the rows the screen samples (a fingerprint)
 *     bound[2..6]  V, r and the address of W2 (the rest of the fingerprint)
 *     bound[7]  a tag, written last
 * Three small launches on `stream`: one pass over W2 (its cost is that of
 * reading W2 once).
 */
#define DSPARK_W2_BOUND_WORDS 8
dspark_status_t dspark_w2_bound(int64_t V, int64_t r, int32_t dtype, const void* W2, uint32_t* bound, void* stream);

/*
 * dspark_head_sample_w2bound -- dspark_head_sample with the bound of
 * dspark_w2_bound (w2_bound: DEVICE, DSPARK_W2_BOUND_WORDS words; NULL makes
 * the call identical to dspark_head_sample).  Same arguments, outputs and
 * rules otherwise.  Only the single-request screen (B = 1, bf16, r = 256)
 * uses the bound; every other shape ignores it.
 *   - Verification: the call uses the bound only when its fingerprint names
 *     this W2 (address, V, r) and the norm of the sampled rows, which the
 *     call measures anyway, equals bound[1].  With a fingerprint for another
 *     W2 the call streams W2 as dspark_head_sample does.  With a matching
 *     address but different sampled rows (W2 changed in place) it proves
 *     nothing from the bound and settles every step with the grid-wide
 *     per-step exchange: correct, slower; path flag 32 of
 *     dspark_workspace_status reports it (16 = the bound was used).
 *   - A change of W2 in place that leaves the sampled rows as they were is
 *     not detected: recompute the bound after every change of W2.
 *   - With a bound that matches, the screen's bound is the measured one,
 *     never looser than the guess dspark_head_sample starts from, so it
 *     proves every step that call proves: the tokens are the same, and conf
 *     and survival are too wherever both calls settle the same steps on the
 *     screen (a step settled by the exchange instead may differ in the last
 *     bits of binary32).
 */
dspark_status_t dspark_head_sample_w2bound(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype,
                                           const void* U, const void* h, const void* W1, const void* W2,
                                           const void* w_conf, float b_conf, const int32_t* x0, const float* gumbel,
                                           const int32_t* force, int32_t* tokens, float* conf, float* survival,
                                           float* logits_out, float* bias_out, const uint32_t* w2_bound,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_head_sample_noalloc -- dspark_head_sample for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and rules as
 * dspark_head_sample, without the workspace: the call uses a static device
 * array of 4 MiB that the library holds on each GPU it runs on until the
 * process ends, zeroes the part it needs at the start of every call (one
 * small fill kernel on `stream`) and calls no allocating routine.
 *   - Shapes whose workspace (dspark_head_sample_workspace_size) exceeds
 *     4 MiB return DSPARK_ERR_WORKSPACE before anything is enqueued (for
 *     example B = 1 any V, or B = 64 with gamma = 7, fit).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     in time on one GPU (different streams, or other threads) race and give
 *     wrong results; serialise them.
 *   - The first call on each device looks the array's device address up
 *     (hipGetSymbolAddress); a failure there returns DSPARK_ERR_HIP.
 */
dspark_status_t dspark_head_sample_noalloc(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                           int32_t dtype, const void* U, const void* h, const void* W1,
                                           const void* W2, const void* w_conf, float b_conf, const int32_t* x0,
                                           const float* gumbel, const int32_t* force, int32_t* tokens, float* conf,
                                           float* survival, float* logits_out, float* bias_out, void* stream);

/*
 * dspark_head_sample_gated -- the same block sampler with the gated Markov
 * head ([W] 3.2, GatedMarkovHead): the previous token's embedding
 * e = W1[x_{k-1}] is gated by the hidden state and itself before the
 * projection,
 *   e'[j]   = e[j] * sigmoid( sum_i Wg[j][i] h[b][k][i] + sum_i Wg[j][H + i] e[i] )
 *   bias[v] = W2[v] . e'
 * (the pages leave the map back to the vocabulary open; this is the vanilla
 * head's W2).  The confidence head still sees e.  Every other argument,
 * output and rule is that of dspark_head_sample.
 *
 *   Wg  [r][H + r] gate weights, columns [h ; W1 row], in the dtype of the others.
 * Workspace: dspark_head_sample_gated_workspace_size bytes, zero-filled before
 * the first use and left zero-filled by every completed call.  The call runs
 * the per-step kernels with one gate launch per step; bf16 with r = 256,
 * B >= 16 and a 16-byte aligned workspace takes the bias on the matrix cores,
 * with e' split into two bf16 operands (hi, and the rounding remainder) so
 * that the bias keeps binary32 accuracy.
 */
dspark_status_t dspark_head_sample_gated(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype,
                                         const void* U, const void* h, const void* W1, const void* W2,
                                         const void* w_conf, const void* Wg, float b_conf, const int32_t* x0,
                                         const float* gumbel, const int32_t* force, int32_t* tokens, float* conf,
                                         float* survival, float* logits_out, float* bias_out, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * dspark_head_sample_rnn -- the same block sampler with the RNN head ([W] 3.2,
 * RNNHead, paper eq. 6): a recurrent state s (s_0 = 0) replaces the embedding
 * in the bias,
 *   z = [s_{k-1} ; W1[x_{k-1}] ; h[b][k]]          (length 2r + H)
 *   u = sigmoid(Wrg z),  s_k = u * s_{k-1} + (1 - u) * tanh(Wrc z)   (elementwise)
 *   bias[v] = W2[v] . s_k
 * (the pages' "(1-sigma)(Wg z)" is read as 1 - sigmoid(Wg z); the map back to
 * the vocabulary as W2).  The confidence head still sees W1[x_{k-1}].  Every
 * other argument, output and rule is that of dspark_head_sample.
 *
 *   Wrg, Wrc  [r][2r + H] update-gate and candidate weights, columns [s ; W1 row ; h],
 *             in the dtype of the others.
 * Workspace: dspark_head_sample_rnn_workspace_size bytes, zero-filled before the
 * first use and left zero-filled by every completed call.  The call runs the
 * per-step kernels with one state launch per step (matrix cores as for
 * dspark_head_sample_gated).
 */
dspark_status_t dspark_head_sample_rnn(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype,
                                       const void* U, const void* h, const void* W1, const void* W2,
                                       const void* w_conf, const void* Wrg, const void* Wrc, float b_conf,
                                       const int32_t* x0, const float* gumbel, const int32_t* force, int32_t* tokens,
                                       float* conf, float* survival, float* logits_out, float* bias_out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_accept_rate -- analytic accept rate per row ([W] 3.3, paper eq. 8):
 *   accept_rate[n] = 1 - 1/2 * || softmax(draft[n, :V]) - softmax(target[n, :V]) ||_1
 * computed in binary32 with max-shifted exponentials.  No clamp is applied:
 * identical rows give exactly 1; rounding can put a result a few 1e-8
 * outside [0, 1].
 *
 *   N >= 0 rows, V >= 1 columns (V < 2^31); dtype of both logit arrays.
 *   draft, target  row n starts at element n * ld (ld >= V); the two strides
 *                  may differ.
 *   accept_rate [N] fp32 out.
 */
dspark_status_t dspark_accept_rate(int64_t N, int64_t V, int32_t dtype, const void* draft, int64_t ld_draft,
                                   const void* target, int64_t ld_target, float* accept_rate, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * dspark_prefix_schedule -- hardware-aware prefix scheduler ([W] 3.3,
 * Algorithm 1).
 *   a[r][j] = conf[r][0] * ... * conf[r][j]   (binary32, left to right)
 *   Sort all B*gamma pairs by (a descending, r ascending, j ascending).
 *   Start from the empty selection: tau = B (one bonus token per request),
 *   Btok = B, Theta_best = B * SPS(B).  Scan the sorted pairs: stop when
 *   Btok + 1 > n_sps; otherwise Theta = (tau + a) * SPS(Btok + 1) in binary64;
 *   accept the pair if Theta > Theta_best (tau += a, Btok += 1,
 *   Theta_best = Theta), else stop.  prefix_len[r] = number of accepted pairs
 *   of request r.  The result equals that sequential binary64 scan bit for bit.
 *
 *   1 <= B <= 8192, gamma >= 0, B * gamma <= 8192.
 *   conf [B][gamma] fp32, values in [0, 1].
 *   sps  [n_sps] fp64, sps[n-1] = SPS(n): the throughput of a verification
 *        batch of n tokens; n_sps >= B.
 *   prefix_len [B] int32 out.
 *   survival_out [B][gamma] fp32 out, optional (NULL = not written).
 *   order_out [B*gamma] int32 out, optional: pair ids r*gamma + j in sorted order.
 *   theta_out [1] fp64 out, optional: Theta_best at the stop.
 *   n_selected_out [1] int32 out, optional: number of accepted pairs.
 */
dspark_status_t dspark_prefix_schedule(int64_t B, int64_t gamma, const float* conf, const double* sps,
                                       int64_t n_sps, int32_t* prefix_len, float* survival_out, int32_t* order_out,
                                       double* theta_out, int32_t* n_selected_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * dspark_verify -- rejection-sampling verification of one draft block per
 * request ([W] 8.2: keep a drafted token with probability
 * min(1, p_target / p_draft); at the first rejection drop it and every later
 * one and draw the next token from the residual max(0, p_target - p_draft);
 * [W] 2.1: after an accepted prefix the target adds one bonus token).
 *
 * For request b with n = n_draft[b] drafted tokens (NULL: n = gamma; values
 * outside [0, gamma] are clamped) and k = 1..n in order, with
 * p_d = softmax(draft[b][k-1][:]) and p_t = softmax(target[b][k-1][:]):
 *   x_k = draft_tokens[b][k-1] is kept iff uniforms[b][k-1] * p_d(x_k) < p_t(x_k)
 *   (a token outside [0, V) is rejected).
 * n_accepted[b] = number of kept tokens.  next_token[b] is drawn with the
 * Gumbel noise row gumbel[b][:]:
 *   after a rejection at position j: argmax over v with p_t(v) > p_d(v) of
 *     ln(p_t(v) - p_d(v)) + gumbel[b][v]   (the residual at position j; with
 *     no such v, the p_t draw below at position j);
 *   if all n are kept: argmax of target[b][n][v] + gumbel[b][v] (the bonus
 *     token from p_t at position n + 1).
 * Probabilities are binary32 with max-shifted exponentials; the argmax takes
 * the lowest id among equal binary32 scores.
 *
 *   B in [0, 65535], gamma in [0, 4096], V >= 1 (V < 2^31); dtype of both
 *   logit arrays.
 *   draft         [B][gamma][V]      draft logits (may be NULL when gamma = 0)
 *   target        [B][gamma + 1][V]  target logits
 *   draft_tokens  [B][gamma] int32
 *   n_draft       [B] int32, optional
 *   uniforms      [B][gamma] fp32 in [0, 1)
 *   gumbel        [B][V] fp32 (e.g. -ln(-ln u))
 *   n_accepted    [B] int32 out;  next_token [B] int32 out
 *   accept_prob   [B][gamma] fp32 out, optional: min(1, p_t(x_k)/p_d(x_k)) for
 *                 k <= n (0 for an invalid token), NaN past n.
 * The workspace (dspark_verify_workspace_size bytes) must be zero-filled
 * before its first use; every completed call leaves it zero-filled again.
 */
dspark_status_t dspark_verify(int64_t B, int64_t gamma, int64_t V, int32_t dtype, const void* draft,
                              const void* target, const int32_t* draft_tokens, const int32_t* n_draft,
                              const float* uniforms, const float* gumbel, int32_t* n_accepted, int32_t* next_token,
                              float* accept_prob, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dspark_block_loss -- the teacher-forced block bias with the joint training
 * loss ([W] 7.2, the joint loss; the training loop's sequential-head step with
 * given previous tokens, [W] 3.2 and paper eq. 5 for the bias).  Positions
 * are [N][gamma] (N anchors, block gamma); for position (n, k), k = 0-based,
 * with x = xp[n][k] and target id y = y[n][k]:
 *   d[v]  = U[n][k][v] + W2[v] . W1[x]                 (draft logits)
 *   ce    = logsumexp(d) - d[y]
 *   l1    = 1/2 sum_v |softmax(d)_v - softmax(t[n][k])_v|,   c* = 1 - l1
 *   conf  = sigmoid(w_conf . [h[n][k]; W1[x]] + b_conf)
 *   bce   = -(c* log conf + (1 - c*) log(1 - conf))
 *   omega = mask[n][k] * exp(-k / decay)   (exp(-(k-1)/decay), k 1-based)
 *   loss  = a_ce L_ce + a_l1 L_l1 + a_conf L_conf,  L_x = sum omega x / sum omega
 * (the pages name the terms, their weights 0.1 / 0.9 / 1.0 and the decay 4.0,
 * not the reduction over positions; the weighted mean is the reading here; 0
 * when no position counts).  A position counts when its mask is non-zero and
 * x and y lie in [0, V); one with x or y out of range gets NaN outputs.
 *
 *   dtype must be DSPARK_BF16 and r must be 256 (the matrix-core tile);
 *   W1 and W2 16-byte aligned; otherwise DSPARK_ERR_BAD_DTYPE / _BAD_SHAPE.
 *   V <= 65535 * 512; decay > 0.
 *   U, t          [N][gamma][V] bf16  draft backbone and target logits
 *   h             [N][gamma][H] bf16  (NULL when H = 0)
 *   W1, W2        [V][256] bf16;  w_conf [H + 256] bf16
 *   xp, y         [N][gamma] int32    given previous tokens, target ids
 *   mask          [N][gamma] fp32, optional (NULL = all ones)
 *   ce, l1, conf, bce  [N][gamma] fp32 out;  loss [4] fp32 out: (L, L_ce, L_l1, L_conf)
 * Workspace: dspark_block_loss_workspace_size bytes, any contents (every word
 * is written before it is read).  Repeated calls give bitwise-identical
 * results (every reduction has a fixed order).
 */
dspark_status_t dspark_block_loss(int64_t N, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype,
                                  const void* U, const void* t, const void* h, const void* W1, const void* W2,
                                  const void* w_conf, float b_conf, const int32_t* xp, const int32_t* y,
                                  const float* mask, float decay, float a_ce, float a_l1, float a_conf, float* ce,
                                  float* l1, float* conf, float* bce, float* loss, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Workspace bytes needed by the entry point of the same name for these
 * shapes; 0 if it needs none.  Pure host functions with no side effects. */
size_t dspark_head_sample_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype);
size_t dspark_head_sample_gated_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                               int32_t dtype);
size_t dspark_head_sample_rnn_workspace_size(int64_t B, int64_t gamma, int64_t V, int64_t H, int64_t r,
                                             int32_t dtype);
size_t dspark_accept_rate_workspace_size(int64_t N, int64_t V, int32_t dtype);
size_t dspark_prefix_schedule_workspace_size(int64_t B, int64_t gamma);
size_t dspark_verify_workspace_size(int64_t B, int64_t gamma, int64_t V, int32_t dtype);
size_t dspark_block_loss_workspace_size(int64_t N, int64_t gamma, int64_t V, int64_t H, int64_t r, int32_t dtype);

/*
 * dspark_workspace_status -- give-up status and path flags of a workspace of
 * dspark_head_sample, dspark_head_sample_gated, dspark_head_sample_rnn,
 * dspark_accept_rate or dspark_verify (each of those workspaces starts with a
 * 256-byte header).  Enqueued on `stream` after the calls to inspect; writes
 * two words to the DEVICE array out[2]:
 *   out[0]  0, or 1 if a bounded wait of some earlier call on this workspace
 *           ran out (see "Persistent kernels and give-ups" above).  It stays
 *           set until the caller zero-fills the workspace.
 *   out[1]  path flags ORed by the calls since the last query, which this
 *           call clears: 1 = the B = 1 candidate screen's guess of the largest
 *           W2 row norm was too small and its step table was rebuilt with the
 *           measured norm; 2 = a B = 1 call settled steps with the grid-wide
 *           per-step exchange; 4 = the batched resident-W2 sampler ran; 8 = the
 *           accept rate's cluster kernel ran; 16 = a B = 1 screen used the
 *           bound of dspark_w2_bound; 32 = that bound's fingerprint did not
 *           match W2 and the block took the exchange.  Diagnostic only: no kernel
 *           reads this word, so its value never affects a result.
 * workspace_bytes >= 256, 256-byte aligned.  Errors as for the other calls.
 */
dspark_status_t dspark_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* out, void* stream);

/*
 * dspark_set_wait_limit -- process-wide number of polls after which every
 * wait for another workgroup gives up, for the calls enqueued after it
 * returns; polls < 0 restores each kernel's default.  polls = 0 makes every
 * such wait give up at once: the kernels still run to completion and report
 * the give-up as described above (a test of the failure path that needs no
 * stalled workgroup).  *previous (optional, host) receives the former value
 * (-1 = defaults).  polls > 2^30 returns DSPARK_ERR_BAD_SHAPE.  This is the
 * library's only mutable global state; it does not affect calls already
 * enqueued.
 */
dspark_status_t dspark_set_wait_limit(int64_t polls, int64_t* previous);

/* Static, NUL-terminated description of a status code. */
const char* dspark_status_string(dspark_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
