"""Pins for the CPU oracle: closed forms, invariants, brute force and
distributional identities that the pages and the mathematics fix.

Each test targets a mistake the oracle could plausibly make (a swapped
factor, the wrong previous token, a missing term, a non-strict comparison,
the wrong tie-break) so that such a mistake fails here.  No test here uses
the GPU.
"""
import itertools

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _sampler_inputs(rng, B, gamma, V, H, r, w_sd=0.5, U_sd=1.0):
    return dict(
        U=rng.normal(0, U_sd, (B, gamma, V)).astype(np.float32),
        h=rng.normal(0, 1, (B, gamma, H)).astype(np.float32),
        W1=rng.normal(0, w_sd, (V, r)).astype(np.float32),
        W2=rng.normal(0, w_sd, (V, r)).astype(np.float32),
        w_conf=rng.normal(0, 0.3, (H + r,)).astype(np.float32),
        b_conf=0.1,
        x0=rng.integers(0, V, B).astype(np.int32),
    )


def _prev_tokens(x0, force):
    """x_{k-1} for every (b, k) when every step is teacher-forced."""
    return np.concatenate([x0[:, None], force[:, :-1]], axis=1)


# ---------------------------------------------------------------------------
# Markov bias (eq. 5) and the step logits
# ---------------------------------------------------------------------------
def test_zero_W2_gives_plain_argmax_of_U():
    rng = _rng(1)
    a = _sampler_inputs(rng, B=3, gamma=4, V=97, H=8, r=6)
    a["W2"][:] = 0
    o = oracle.head_sample(**a, want_logits=True)
    assert np.all(o["bias"] == 0.0)
    np.testing.assert_array_equal(o["logits"], a["U"].astype(np.float64))
    np.testing.assert_array_equal(o["tokens"], np.argmax(a["U"], axis=2))


def test_one_hot_factors_give_indicator_bias():
    # W1[v] = e_f(v), W2[v] = e_g(v)  =>  bias[v] = [g(v) == f(x_{k-1})].
    # f != g, so swapping the roles of W1 and W2 gives a different answer.
    V, r, B, gamma = 40, 7, 2, 5
    f = (np.arange(V) * 3) % r
    g = (np.arange(V) * 5 + 1) % r
    W1 = np.zeros((V, r), np.float32)
    W2 = np.zeros((V, r), np.float32)
    W1[np.arange(V), f] = 1
    W2[np.arange(V), g] = 1
    rng = _rng(2)
    x0 = np.array([3, 17], np.int32)
    force = rng.integers(0, V, (B, gamma)).astype(np.int32)
    o = oracle.head_sample(U=np.zeros((B, gamma, V), np.float32), h=np.zeros((B, gamma, 1), np.float32),
                           W1=W1, W2=W2, w_conf=np.zeros(1 + r, np.float32), b_conf=0.0, x0=x0, force=force,
                           want_logits=True)
    prev = _prev_tokens(x0, force)
    expect = (g[None, None, :] == f[prev][:, :, None]).astype(np.float64)
    np.testing.assert_array_equal(o["bias"], expect)


def test_bias_is_W2_times_previous_W1_row():
    # library matmul against the oracle's loops, previous tokens pinned by force
    rng = _rng(3)
    a = _sampler_inputs(rng, B=2, gamma=6, V=53, H=5, r=9)
    force = rng.integers(0, 53, (2, 6)).astype(np.int32)
    o = oracle.head_sample(**a, force=force, want_logits=True)
    prev = _prev_tokens(a["x0"], force)
    W1 = a["W1"].astype(np.float64)
    W2 = a["W2"].astype(np.float64)
    for b in range(2):
        for k in range(6):
            ref = W2 @ W1[prev[b, k]]
            np.testing.assert_allclose(o["bias"][b, k], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(o["logits"][b, k], a["U"][b, k] + ref, rtol=1e-12, atol=1e-14)


def test_bigram_walk_worked_by_hand():
    # U = 0, W1 = identity, W2 = permutation matrix with W2[pi(x), x] = 1: the
    # greedy chain follows pi.  pi = 0->2, 1->4, 2->1, 3->0, 4->3.
    pi = [2, 4, 1, 0, 3]
    V = 5
    W1 = np.eye(V, dtype=np.float32)
    W2 = np.zeros((V, V), np.float32)
    for x, y in enumerate(pi):
        W2[y, x] = 1.0
    o = oracle.head_sample(U=np.zeros((2, 6, V), np.float32), h=np.zeros((2, 6, 1), np.float32), W1=W1, W2=W2,
                           w_conf=np.zeros(1 + V, np.float32), b_conf=0.0, x0=np.array([0, 3], np.int32))
    np.testing.assert_array_equal(o["tokens"][0], [2, 1, 4, 3, 0, 2])
    np.testing.assert_array_equal(o["tokens"][1], [0, 2, 1, 4, 3, 0])


def test_all_equal_scores_pick_lowest_token():
    V = 31
    o = oracle.head_sample(U=np.full((2, 3, V), 0.25, np.float32), h=np.zeros((2, 3, 2), np.float32),
                           W1=np.ones((V, 4), np.float32), W2=np.zeros((V, 4), np.float32),
                           w_conf=np.zeros(6, np.float32), b_conf=0.0, x0=np.array([5, 30], np.int32))
    assert np.all(o["tokens"] == 0)
    assert np.all(o["margin"] == 0.0)


def test_decision_is_taken_in_binary32():
    # Two scores differing by less than half a binary32 ulp at 1.0 round to
    # the same float, so the lower token id wins the argmax.  The fp64
    # margin still reports the difference.
    V = 4
    U = np.zeros((1, 1, V), np.float32)
    U[0, 0, 1] = 1.0
    U[0, 0, 3] = 1.0
    W1 = np.ones((V, 1), np.float32)
    W2 = np.zeros((V, 1), np.float32)
    W2[3, 0] = 2.0**-30  # token 3 larger by 2^-30 in fp64, equal in binary32
    o = oracle.head_sample(U=U, h=np.zeros((1, 1, 1), np.float32), W1=W1, W2=W2, w_conf=np.zeros(2, np.float32),
                           b_conf=0.0, x0=np.array([0], np.int32))
    assert o["tokens"][0, 0] == 1
    assert o["margin"][0, 0] == pytest.approx(2.0**-30, rel=1e-9)


def test_bf16_inputs_are_widened_exactly():
    # values exactly representable in bfloat16 give identical results in both dtypes
    rng = _rng(4)
    a = _sampler_inputs(rng, B=2, gamma=3, V=64, H=6, r=8)
    for k in ("U", "h", "W1", "W2", "w_conf"):
        a[k] = np.round(a[k] * 16) / 16  # few mantissa bits: exact in bf16
    o32 = oracle.head_sample(**a, want_logits=True)
    a16 = dict(a)
    for k in ("U", "h", "W1", "W2", "w_conf"):
        a16[k] = synth.f32_to_bf16(a[k])
        assert np.array_equal(synth.bf16_to_f32(a16[k]), a[k])
    o16 = oracle.head_sample(**a16, want_logits=True)
    for k in ("tokens", "conf", "survival", "logits", "bias"):
        np.testing.assert_array_equal(o32[k], o16[k])


def test_gumbel_max_draws_follow_the_softmax_chain():
    # Gumbel-max is an exact sampler of softmax(logits); across two dependent
    # steps the sequence (x1, x2) has probability
    # softmax(U_1 + W2 W1[x0])[x1] * softmax(U_2 + W2 W1[x1])[x2].
    rng = _rng(5)
    V, r, gamma, n = 4, 2, 2, 200_000
    U1 = rng.normal(0, 1, (gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 1, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 1, (V, r)).astype(np.float32)
    x0 = 2
    U = np.broadcast_to(U1, (n, gamma, V)).copy()
    G = synth.gumbel(synth.key(77, 1), (n, gamma, V))
    o = oracle.head_sample(U=U, h=np.zeros((n, gamma, 1), np.float32), W1=W1, W2=W2,
                           w_conf=np.zeros(1 + r, np.float32), b_conf=0.0, x0=np.full(n, x0, np.int32), gumbel=G)
    W1d, W2d = W1.astype(np.float64), W2.astype(np.float64)
    p1 = special.softmax(U1[0] + W2d @ W1d[x0])
    prob = np.array([p1[a] * special.softmax(U1[1] + W2d @ W1d[a])[b] for a in range(V) for b in range(V)])
    counts = np.bincount(o["tokens"][:, 0] * V + o["tokens"][:, 1], minlength=V * V)
    chi2 = np.sum((counts - n * prob) ** 2 / (n * prob))
    assert stats.chi2.sf(chi2, df=V * V - 1) > 1e-3, chi2


# ---------------------------------------------------------------------------
# Confidence head and survival
# ---------------------------------------------------------------------------
def test_confidence_closed_forms():
    rng = _rng(6)
    B, gamma, V, H, r = 2, 5, 30, 7, 4
    a = _sampler_inputs(rng, B, gamma, V, H, r)
    force = rng.integers(0, V, (B, gamma)).astype(np.int32)
    prev = _prev_tokens(a["x0"], force)

    a0 = dict(a, w_conf=np.zeros(H + r, np.float32), b_conf=0.3)
    o = oracle.head_sample(**a0, force=force)
    np.testing.assert_allclose(o["conf"], special.expit(0.3), rtol=1e-15)

    i = 4  # one-hot on the hidden part picks h[b, k, i]
    w = np.zeros(H + r, np.float32)
    w[i] = 1.0
    o = oracle.head_sample(**dict(a, w_conf=w, b_conf=-0.2), force=force)
    np.testing.assert_allclose(o["conf"], special.expit(a["h"][:, :, i].astype(np.float64) - 0.2), rtol=1e-14)

    j = 2  # one-hot on the Markov part picks W1[x_{k-1}, j]: the PREVIOUS token
    w = np.zeros(H + r, np.float32)
    w[H + j] = 1.0
    o = oracle.head_sample(**dict(a, w_conf=w, b_conf=0.5), force=force)
    np.testing.assert_allclose(o["conf"], special.expit(a["W1"][prev, j].astype(np.float64) + 0.5), rtol=1e-14)


def test_survival_is_running_product_of_conf():
    rng = _rng(7)
    a = _sampler_inputs(rng, B=3, gamma=9, V=41, H=6, r=5)
    o = oracle.head_sample(**a)
    np.testing.assert_allclose(o["survival"], np.cumprod(o["conf"], axis=1), rtol=1e-15)
    assert np.all(o["survival"][:, 0] == o["conf"][:, 0])
    assert np.all(np.diff(o["survival"], axis=1) <= 0)
    assert np.all((o["survival"] > 0) & (o["survival"] <= 1))


def test_force_feeds_the_next_step_but_not_the_reported_token():
    rng = _rng(8)
    a = _sampler_inputs(rng, B=1, gamma=4, V=23, H=3, r=4, w_sd=1.0)
    free = oracle.head_sample(**a)
    force = np.full((1, 4), -1, np.int32)
    alt = (free["tokens"][0, 0] + 7) % 23
    force[0, 0] = alt
    forced = oracle.head_sample(**a, force=force)
    assert forced["tokens"][0, 0] == free["tokens"][0, 0]  # step 1 still reports its own sample
    # step 2 onwards continues from the forced token: same as a fresh call whose anchor is it
    a2 = dict(a, U=a["U"][:, 1:], h=a["h"][:, 1:], x0=np.array([alt], np.int32))
    tail = oracle.head_sample(**a2)
    np.testing.assert_array_equal(forced["tokens"][:, 1:], tail["tokens"])


# ---------------------------------------------------------------------------
# Analytic accept rate (eq. 8)
# ---------------------------------------------------------------------------
def test_accept_rate_identical_rows_is_exactly_one():
    rng = _rng(9)
    d = rng.normal(0, 3, (5, 300)).astype(np.float32)
    np.testing.assert_array_equal(oracle.accept_rate(d, d.copy()), 1.0)
    db = synth.f32_to_bf16(d)
    np.testing.assert_array_equal(oracle.accept_rate(db, db.copy()), 1.0)


def test_accept_rate_shift_invariance():
    rng = _rng(10)
    d = (np.round(rng.normal(0, 2, (4, 200)) * 64) / 64).astype(np.float32)
    t = d + np.float32(3.0)  # exact in binary32 for these values
    np.testing.assert_allclose(oracle.accept_rate(d, t), 1.0, atol=1e-13)


def test_accept_rate_two_token_closed_form():
    rng = _rng(11)
    d = rng.normal(0, 2, (50, 2)).astype(np.float32)
    t = rng.normal(0, 2, (50, 2)).astype(np.float32)
    d64, t64 = d.astype(np.float64), t.astype(np.float64)
    ref = 1 - np.abs(special.expit(d64[:, 1] - d64[:, 0]) - special.expit(t64[:, 1] - t64[:, 0]))
    np.testing.assert_allclose(oracle.accept_rate(d, t), ref, atol=1e-14)


def test_accept_rate_equals_rejection_sampling_acceptance():
    # Verification accepts a draft token x ~ p_d with probability
    # min(1, p_t(x)/p_d(x)); its expectation is the accept rate.
    rng = _rng(12)
    d = rng.normal(0, 2, (8, 500)).astype(np.float32)
    t = (0.8 * d + rng.normal(0, 1.5, d.shape)).astype(np.float32)
    p = special.softmax(d.astype(np.float64), axis=1)
    q = special.softmax(t.astype(np.float64), axis=1)
    expect = np.sum(p * np.minimum(1.0, q / p), axis=1)
    cs, sm = oracle.accept_rate(d, t, with_summin=True)
    np.testing.assert_allclose(cs, expect, atol=1e-12)
    np.testing.assert_allclose(sm, expect, atol=1e-12)


def test_accept_rate_monte_carlo_of_the_verify_rule():
    rng = _rng(13)
    V, n = 6, 400_000
    d = rng.normal(0, 1, (1, V)).astype(np.float32)
    t = rng.normal(0, 1, (1, V)).astype(np.float32)
    p = special.softmax(d[0].astype(np.float64))
    q = special.softmax(t[0].astype(np.float64))
    x = rng.choice(V, size=n, p=p)
    acc = rng.random(n) < np.minimum(1.0, q[x] / p[x])
    c = oracle.accept_rate(d, t)[0]
    assert abs(acc.mean() - c) < 5 * np.sqrt(c * (1 - c) / n)


def test_accept_rate_disjoint_and_bounds_and_symmetry():
    d = np.full((1, 10), -60.0, np.float32)
    t = np.full((1, 10), -60.0, np.float32)
    d[0, 2] = 60.0
    t[0, 7] = 60.0
    assert oracle.accept_rate(d, t)[0] < 1e-40
    rng = _rng(14)
    d = rng.normal(0, 4, (20, 333)).astype(np.float32)
    t = rng.normal(0, 4, (20, 333)).astype(np.float32)
    c1 = oracle.accept_rate(d, t)
    assert np.all(c1 >= -1e-15) and np.all(c1 <= 1 + 1e-15)
    np.testing.assert_allclose(oracle.accept_rate(t, d), c1, atol=1e-15)
    perm = rng.permutation(333)
    np.testing.assert_allclose(oracle.accept_rate(d[:, perm], t[:, perm]), c1, atol=1e-13)


def test_accept_rate_row_stride():
    rng = _rng(15)
    V, ld = 70, 96
    d = rng.normal(0, 2, (6, ld)).astype(np.float32)
    t = rng.normal(0, 2, (6, ld)).astype(np.float32)
    d[:, V:] = 1e30  # padding beyond V is never read
    t[:, V:] = -1e30
    ref = oracle.accept_rate(np.ascontiguousarray(d[:, :V]), np.ascontiguousarray(t[:, :V]))
    np.testing.assert_array_equal(oracle.accept_rate(d, t, V=V), ref)


# ---------------------------------------------------------------------------
# Prefix scheduler (Algorithm 1)
# ---------------------------------------------------------------------------
def test_schedule_worked_by_hand():
    conf = np.array([[0.9, 0.5], [0.8, 0.8]], np.float32)
    sps = np.array([1.0, 1.0, 0.9, 0.8, 0.7, 0.5])
    # survivals: (0,1) 0.9, (1,1) 0.8, (1,2) 0.64, (0,2) 0.45
    # Theta0 = 2*1.0; 2.9*0.9 = 2.61 > 2; 3.7*0.8 = 2.96 > 2.61;
    # 4.34*0.7 = 3.038 > 2.96; 4.79*0.5 = 2.395 -> stop
    o = oracle.prefix_schedule(conf, sps)
    np.testing.assert_array_equal(o["prefix_len"], [1, 2])
    np.testing.assert_array_equal(o["order"], [0, 2, 3, 1])
    assert o["n_selected"] == 3
    assert o["theta"] == pytest.approx(3.038, abs=1e-6)
    # a table of 4 entries caps the batch at 4 tokens: 2 pairs only
    o = oracle.prefix_schedule(conf, sps[:4])
    np.testing.assert_array_equal(o["prefix_len"], [1, 1])
    assert o["theta"] == pytest.approx(2.96, abs=1e-6)


def test_schedule_strict_improvement_and_empty_selection():
    # equal Theta stops the scan
    o = oracle.prefix_schedule(np.array([[1.0, 0.0]], np.float32), np.ones(3))
    np.testing.assert_array_equal(o["prefix_len"], [1])
    assert o["theta"] == 2.0
    # a first pair that lowers Theta leaves every request at length 0
    o = oracle.prefix_schedule(np.array([[0.5, 0.5], [0.5, 0.5]], np.float32), np.array([1.0, 3.0, 0.1, 0.1, 0.1]))
    np.testing.assert_array_equal(o["prefix_len"], [0, 0])
    assert o["theta"] == 6.0 and o["n_selected"] == 0


def test_schedule_tie_order_and_fp32_survival():
    conf = np.full((3, 2), 0.5, np.float32)
    o = oracle.prefix_schedule(conf, np.ones(10))
    np.testing.assert_array_equal(o["order"], [0, 2, 4, 1, 3, 5])
    rng = _rng(16)
    conf = rng.random((7, 9)).astype(np.float32)
    o = oracle.prefix_schedule(conf, np.ones(80))
    np.testing.assert_array_equal(o["survival"], np.cumprod(conf, axis=1, dtype=np.float32))


def _exhaustive_best(conf, sps):
    B, gamma = conf.shape
    a = np.cumprod(conf, axis=1, dtype=np.float32).astype(np.float64)
    best = -np.inf
    for ell in itertools.product(range(gamma + 1), repeat=B):
        n = B + sum(ell)
        if n > len(sps):
            continue
        tau = B + sum(a[r, :l].sum() for r, l in enumerate(ell))
        best = max(best, tau * sps[n - 1])
    return best


def test_schedule_matches_exhaustive_search_for_step_rate_tables():
    # With SPS(n) = 1/(alpha + beta n) the throughput of the best selection of
    # n pairs is unimodal in n, so the greedy scan's first stop is the global
    # optimum over every choice of prefix lengths.
    rng = _rng(17)
    for trial in range(150):
        B, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        conf = (1 / (1 + np.exp(-rng.normal(1.0, 1.5, (B, gamma))))).astype(np.float32)
        alpha, beta = rng.uniform(0.5, 3.0), rng.uniform(0.01, 1.5)
        n_sps = B * (gamma + 1) + int(rng.integers(0, 3))
        sps = 1.0 / (alpha + beta * np.arange(1, n_sps + 1))
        o = oracle.prefix_schedule(conf, sps)
        best = _exhaustive_best(conf, sps)
        assert o["theta"] == pytest.approx(best, rel=1e-12), trial
        a = np.cumprod(conf, axis=1, dtype=np.float32).astype(np.float64)
        ell = o["prefix_len"]
        tau = B + sum(a[r, :l].sum() for r, l in enumerate(ell))
        assert tau * sps[B + ell.sum() - 1] == pytest.approx(o["theta"], rel=1e-12)


def test_schedule_increasing_table_takes_every_pair_up_to_capacity():
    s = synth.SCHEDULE_TRAIN
    conf = synth.schedule_conf(s)
    o = oracle.prefix_schedule(conf, synth.sps_table(s.n_sps, "tokens"))
    # SPS(n) = n/(2 + 0.004 n) increases, so every pair improves Theta until
    # the table runs out at Btok = n_sps.
    assert o["n_selected"] == min(s.B * s.gamma, s.n_sps - s.B)
    surv = o["survival"].reshape(-1)
    chosen = o["order"][: o["n_selected"]]
    rest = o["order"][o["n_selected"]:]
    assert surv[chosen].min() >= surv[rest].max()


def test_schedule_invariants_on_training_workload():
    s = synth.SCHEDULE_TRAIN
    conf = synth.schedule_conf(s)
    o = oracle.prefix_schedule(conf, synth.sps_table(s.n_sps, "steps"))
    ell, order = o["prefix_len"], o["order"]
    assert np.array_equal(np.sort(order), np.arange(s.B * s.gamma))
    surv = o["survival"].reshape(-1)
    assert np.all(np.diff(surv[order]) <= 0)
    assert ell.sum() == o["n_selected"] and np.all((ell >= 0) & (ell <= s.gamma))
    sel = order[: o["n_selected"]]
    for pid in sel:  # every selected (r, j) has (r, j' < j) selected too
        r, j = divmod(int(pid), s.gamma)
        assert j < ell[r]
    assert 0 < o["n_selected"] < s.B * s.gamma  # the step-rate curve stops early


# ---------------------------------------------------------------------------
# rejection-sampling verification ([W] 8.2)
# ---------------------------------------------------------------------------
def _softmax64(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _emitted(out, x, n):
    """The emitted sequence of each request: accepted drafts, then the sample."""
    seqs = []
    for b in range(len(out["n_acc"])):
        a = int(out["n_acc"][b])
        seqs.append(list(x[b, :a]) + [int(out["next_token"][b])])
    return seqs


@pytest.mark.parametrize("gamma", [1, 2])
def test_verify_emits_the_target_distribution(gamma):
    """The theorem [W] 8.2 states: with x_k ~ p_d, the first emitted token
    follows p_t at position 1 exactly, and given x_1 accepted the next
    emitted token follows p_t at position 2.  Chi-square over 240,000
    Monte Carlo draws (drafts from numpy's sampler, not the oracle's)."""
    rng = _rng(81 + gamma)
    V, M = 4, 240_000
    d1 = rng.normal(0, 1.2, (gamma, V))
    t1 = rng.normal(0, 1.2, (gamma + 1, V))
    pd, pt = _softmax64(d1), _softmax64(t1)
    x = np.stack([rng.choice(V, size=M, p=pd[k]) for k in range(gamma)], axis=1).astype(np.int32)
    d = np.broadcast_to(d1.astype(np.float32), (M, gamma, V))
    t = np.broadcast_to(t1.astype(np.float32), (M, gamma + 1, V))
    u = rng.random((M, gamma)).astype(np.float32)
    G = rng.gumbel(size=(M, V)).astype(np.float32)
    out = oracle.verify(d, t, x, u, G)
    seqs = _emitted(out, x, gamma)
    first = np.array([s[0] for s in seqs])
    counts = np.bincount(first, minlength=V)
    chi2 = np.sum((counts - M * pt[0]) ** 2 / (M * pt[0]))
    assert stats.chi2.sf(chi2, df=V - 1) > 1e-3, (chi2, counts / M, pt[0])
    # second emitted token given the first draft was accepted
    acc = out["n_acc"] >= 1
    second = np.array([s[1] for s, a in zip(seqs, acc) if a])
    m = len(second)
    counts2 = np.bincount(second, minlength=V)
    chi2 = np.sum((counts2 - m * pt[1]) ** 2 / (m * pt[1]))
    assert stats.chi2.sf(chi2, df=V - 1) > 1e-3, (chi2, counts2 / m, pt[1])
    # the acceptance frequency of x_1 is sum_v min(p_d, p_t) (the accept rate)
    assert abs(acc.mean() - np.minimum(pd[0], pt[0]).sum()) < 4e-3


def test_verify_worked_by_hand():
    """V = 3, p_d = (0.5, 0.3, 0.2), p_t = (0.2, 0.3, 0.5), x_1 = 0:
    accept iff u < 0.4; the residual max(0, p_t - p_d) = (0, 0, 0.3) leaves
    token 2 whatever the noise."""
    ld = np.log([0.5, 0.3, 0.2]).astype(np.float32)
    lt = np.log([0.2, 0.3, 0.5]).astype(np.float32)
    d = np.tile(ld, (3, 1, 1))
    t = np.stack([np.stack([lt, lt])] * 3)  # position 2 = the same distribution
    x = np.zeros((3, 1), np.int32)
    u = np.array([[0.3], [0.5], [0.39]], np.float32)
    G = np.array([[9.0, 0.0, 0.0], [9.0, 0.0, 0.0], [0.0, 0.0, 9.0]], np.float32)
    out = oracle.verify(d, t, x, u, G)
    assert list(out["n_acc"]) == [1, 0, 1]
    np.testing.assert_allclose(out["accept_prob"][:, 0], 0.4, rtol=1e-6)
    assert out["next_token"][1] == 2 and out["residual"][1] == 1  # residual: token 2 only
    # accepted: bonus = argmax(t[1] + G): token 0 for row 0 (log .2 + 9), token 2 for row 2
    assert out["next_token"][0] == 0 and out["next_token"][2] == 2
    assert list(out["sample_pos"]) == [1, 0, 1]


def test_verify_identical_distributions_accept_everything():
    rng = _rng(90)
    B, gamma, V = 6, 5, 37
    t = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    d = np.ascontiguousarray(t[:, :gamma])
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    u = (rng.random((B, gamma)) * 0.999).astype(np.float32)
    G = rng.gumbel(size=(B, V)).astype(np.float32)
    n = np.array([5, 4, 0, 1, 3, 5], np.int32)
    out = oracle.verify(d, t, x, u, G, n_draft=n)
    assert np.array_equal(out["n_acc"], n)
    bonus = np.argmax(t[np.arange(B), n] + G, axis=1)  # float32 scores
    assert np.array_equal(out["next_token"], bonus)
    assert np.array_equal(out["sample_pos"], n) and not out["residual"].any()
    for b in range(B):
        np.testing.assert_allclose(out["accept_prob"][b, : n[b]], 1.0)
        assert np.all(np.isnan(out["accept_prob"][b, n[b]:]))


def test_verify_rejections_zero_target_invalid_token_and_empty_residual():
    rng = _rng(91)
    B, gamma, V = 4, 3, 16
    t = rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)
    d = np.ascontiguousarray(t[:, :gamma]).copy()
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    u = np.full((B, gamma), 0.5, np.float32)
    G = rng.gumbel(size=(B, V)).astype(np.float32)
    t[0, 1, x[0, 1]] = -np.inf        # p_t(x) = 0: rejected at position 2, even for u = 0
    u[0, 1] = 0.0                     # (0 * p_d < 0 is false: the test is strict)
    x[1, 0] = V                       # out of range: rejected at position 1
    x[2, 2] = -1                      # rejected at position 3
    d[3, 0, :] = rng.normal(0, 1, V)  # differs: a real residual exists at position 1
    u[3, 0] = 0.99999
    out = oracle.verify(d, t, x, u, G)
    assert out["n_acc"][0] == 1 and out["sample_pos"][0] == 1 and out["accept_prob"][0, 1] == 0.0
    # probabilities past the rejection are still reported, none past n
    assert np.all(np.isfinite(out["accept_prob"])) and out["accept_prob"][1, 0] == 0.0
    # d == t at the rejected positions of requests 1 and 2: the residual is empty,
    # so the sample falls back to p_t there
    for b, k in ((1, 0), (2, 2)):
        assert out["n_acc"][b] == k and out["residual"][b] == 0
        assert out["next_token"][b] == np.argmax(t[b, k] + G[b])
    # request 0: removing x's target mass raises every other p_t above p_d, so
    # the residual is p_t - p_d on all tokens but x
    assert out["residual"][0] == 1 and out["next_token"][0] != x[0, 1]
    r = _softmax64(t[0, 1]) - _softmax64(d[0, 1])
    sc = np.where(r > 0, np.log(np.where(r > 0, r, 1)) + G[0], -np.inf).astype(np.float32)
    assert out["next_token"][0] == int(np.argmax(sc))
    # request 3: if x_1 was rejected, the sample lies where p_t > p_d
    if out["n_acc"][3] == 0:
        assert out["residual"][3] == 1
        v = out["next_token"][3]
        assert _softmax64(t[3, 0])[v] > _softmax64(d[3, 0])[v]


def test_verify_residual_sample_is_gumbel_max_of_log_residual():
    """Brute force of the residual draw on one rejected position."""
    rng = _rng(92)
    V = 50
    d = rng.normal(0, 1, (1, 1, V)).astype(np.float32)
    t = rng.normal(0, 1, (1, 2, V)).astype(np.float32)
    pd, pt = _softmax64(d[0, 0]), _softmax64(t[0, 0])
    x = np.array([[int(np.argmax(pd / pt))]], np.int32)  # the least acceptable token
    u = np.array([[0.999]], np.float32)
    for seed in range(20):
        G = rng.gumbel(size=(1, V)).astype(np.float32)
        out = oracle.verify(d, t, x, u, G)
        assert out["n_acc"][0] == 0 and out["residual"][0] == 1
        r = pt - pd
        sc = np.where(r > 0, np.log(np.where(r > 0, r, 1)) + G[0], -np.inf).astype(np.float32)
        assert out["next_token"][0] == int(np.argmax(sc)), seed


# ---------------------------------------------------------------------------
# gated Markov head ([W] 3.2): bias = W2 . (sigmoid(Wg [h_k; e]) * e)
# ---------------------------------------------------------------------------
def test_gated_zero_gate_weights_halve_the_bias():
    """Wg = 0 makes every gate 1/2: the gated head is the vanilla head with
    W2 / 2 (both scalings are exact)."""
    rng = _rng(120)
    p = _sampler_inputs(rng, B=3, gamma=4, V=300, H=12, r=8)
    Wg = np.zeros((8, 12 + 8), np.float32)
    g = oracle.head_sample(**p, Wg=Wg, want_logits=True)
    v = oracle.head_sample(**{**p, "W2": p["W2"] * np.float32(0.5)}, want_logits=True)
    assert np.array_equal(g["tokens"], v["tokens"])
    assert np.array_equal(g["bias"], v["bias"])
    assert np.array_equal(g["conf"], v["conf"])  # the confidence head sees e, not the gated e


def test_gated_saturated_gate_is_the_vanilla_head():
    """Positive embeddings and Wg = [0 | c I] with c e_j > 60 put every gate
    within 1e-26 of 1."""
    rng = _rng(121)
    p = _sampler_inputs(rng, B=2, gamma=5, V=400, H=6, r=8)
    p["W1"] = (np.abs(p["W1"]) + np.float32(0.5)).astype(np.float32)
    Wg = np.zeros((8, 6 + 8), np.float32)
    Wg[:, 6:] = np.eye(8, dtype=np.float32) * np.float32(200.0)
    g = oracle.head_sample(**p, Wg=Wg, want_logits=True)
    v = oracle.head_sample(**p, want_logits=True)
    assert np.array_equal(g["tokens"], v["tokens"])
    np.testing.assert_allclose(g["bias"], v["bias"], rtol=1e-12, atol=1e-14)


def test_gated_hidden_state_switches_each_position():
    """A gate driven only by the mean of h_k: h_k = +100 opens it (the vanilla
    token), h_k = -100 closes it (bias ~ 1e-44: the plain argmax of U_k).
    Teacher forcing fixes every previous token, so each position is checked
    on its own; a wrong position index for h fails here."""
    rng = _rng(122)
    B, gamma, V, H, r = 2, 6, 500, 10, 8
    p = _sampler_inputs(rng, B=B, gamma=gamma, V=V, H=H, r=r, w_sd=2.0, U_sd=0.5)
    sign = np.array([[1, -1, -1, 1, 1, -1], [-1, 1, -1, 1, -1, 1]], np.float32)
    p["h"] = np.repeat((100.0 * sign)[:, :, None], H, axis=2).astype(np.float32)
    Wg = np.zeros((r, H + r), np.float32)
    Wg[:, :H] = np.float32(1.0 / H)
    force = rng.integers(0, V, (B, gamma)).astype(np.int32)
    g = oracle.head_sample(**p, force=force, Wg=Wg)
    v = oracle.head_sample(**p, force=force)
    plain = np.argmax(p["U"], axis=2)
    on = sign > 0
    assert np.array_equal(g["tokens"][on], v["tokens"][on])
    assert np.array_equal(g["tokens"][~on], plain[~on])
    assert not np.array_equal(v["tokens"][~on], plain[~on])  # the bias matters in this setting


# ---------------------------------------------------------------------------
# RNN head ([W] 3.2, paper eq. 6): s_k = u s_{k-1} + (1 - u) tanh(Wc z),
# u = sigmoid(Wg z), z = [s_{k-1}; e; h_k], s_0 = 0, bias = W2 . s_k
# ---------------------------------------------------------------------------
def _rnn_setup(seed, B=2, gamma=5, V=400, H=10, r=8):
    rng = _rng(seed)
    p = _sampler_inputs(rng, B=B, gamma=gamma, V=V, H=H, r=r, w_sd=0.5, U_sd=0.3)
    p["W1"] = (np.abs(p["W1"]) + np.float32(0.5)).astype(np.float32)  # e_j >= 0.5
    force = rng.integers(0, V, (B, gamma)).astype(np.int32)
    Z = 2 * r + H
    return p, force, np.zeros((r, Z), np.float32), np.zeros((r, Z), np.float32)


def _expected_tokens(U, bias_rows):
    """argmax of the binary32 score U + bias per (request, position)."""
    return np.argmax((U.astype(np.float64) + bias_rows).astype(np.float32), axis=2)


def test_rnn_zero_weights_give_no_bias():
    p, force, Wrg, Wrc = _rnn_setup(130)
    out = oracle.head_sample(**p, force=force, Wr=(Wrg, Wrc), want_logits=True)
    assert np.all(out["bias"] == 0.0)  # u = 1/2, tanh(0) = 0: the state stays 0
    assert np.array_equal(out["tokens"], np.argmax(p["U"], axis=2))


def test_rnn_recurrence_is_geometric():
    """u = 1/2 and a saturated candidate (tanh(200 e) = 1): s_k = 1 - 2^-k."""
    p, force, Wrg, Wrc = _rnn_setup(131)
    r = 8
    Wrc[:, r:2 * r] = np.eye(r, dtype=np.float32) * np.float32(200.0)
    out = oracle.head_sample(**p, force=force, Wr=(Wrg, Wrc), want_logits=True)
    rows = p["W2"].astype(np.float64).sum(axis=1)
    k = np.arange(1, 6)
    want = (1.0 - 2.0 ** -k)[None, :, None] * rows[None, None, :]
    np.testing.assert_allclose(out["bias"], np.broadcast_to(want, out["bias"].shape), rtol=1e-12, atol=1e-12)
    assert np.array_equal(out["tokens"], _expected_tokens(p["U"], want))


def test_rnn_closed_update_gate_follows_h_of_each_position():
    """u ~ 0 (sigmoid(-200 e)) and a candidate driven by the mean of h_k:
    h_k = +-100 gives s_k = +-1, bias = +-rowsum(W2), position by position."""
    p, force, Wrg, Wrc = _rnn_setup(132, H=10)
    r, H = 8, 10
    Wrg[:, r:2 * r] = -np.eye(r, dtype=np.float32) * np.float32(200.0)
    Wrc[:, 2 * r:] = np.float32(1.0 / H)
    sign = np.array([[1, -1, 1, 1, -1], [-1, -1, 1, -1, 1]], np.float64)
    p["h"] = np.repeat((100.0 * sign)[:, :, None], H, axis=2).astype(np.float32)
    out = oracle.head_sample(**p, force=force, Wr=(Wrg, Wrc), want_logits=True)
    rows = p["W2"].astype(np.float64).sum(axis=1)
    want = sign[:, :, None] * rows[None, None, :]
    np.testing.assert_allclose(out["bias"], want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out["tokens"], _expected_tokens(p["U"], want))


def test_rnn_state_feeds_the_next_step():
    """u ~ 0, candidate = tanh(1000 s_{k-1} + mean(h_k)): h_1 = +100 sets s_1 = 1
    and the state alone keeps it at 1 (h_k = 0 afterwards); without s in z it
    would fall back to 0."""
    p, force, Wrg, Wrc = _rnn_setup(133, H=10)
    r, H = 8, 10
    Wrg[:, r:2 * r] = -np.eye(r, dtype=np.float32) * np.float32(200.0)
    Wrc[:, :r] = np.eye(r, dtype=np.float32) * np.float32(1000.0)
    Wrc[:, 2 * r:] = np.float32(1.0 / H)
    h = np.zeros_like(p["h"])
    h[:, 0, :] = 100.0
    p["h"] = h
    out = oracle.head_sample(**p, force=force, Wr=(Wrg, Wrc), want_logits=True)
    rows = p["W2"].astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(out["bias"], np.broadcast_to(rows, out["bias"].shape), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Teacher-forced block bias with the joint loss ([W] section 7.2): pinned by
# closed forms, by the accept-rate oracle, and by the binary entropy.
# ---------------------------------------------------------------------------
def _bl_inputs(N, gamma, V, H, r, seed=0):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(U=f(N, gamma, V), t=f(N, gamma, V), h=f(N, gamma, H), W1=f(V, r), W2=f(V, r), w_conf=f(H + r),
                b_conf=0.0, xp=rng.integers(0, V, (N, gamma)).astype(np.int32),
                y=rng.integers(0, V, (N, gamma)).astype(np.int32))


def test_block_loss_uniform_draft_closed_form():
    """W2 = 0 and U = 0 make the draft uniform: CE = log V; t = U gives L1 = 0,
    c* = 1; w = 0, b = 0 give conf = 1/2 and BCE = log 2."""
    V = 37
    x = _bl_inputs(2, 3, V, 4, 5)
    x.update(U=np.zeros((2, 3, V), np.float32), t=np.zeros((2, 3, V), np.float32),
             W2=np.zeros((V, 5), np.float32), w_conf=np.zeros(9, np.float32))
    o = oracle.block_loss(**x)
    np.testing.assert_allclose(o["ce"], np.log(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["l1"], 0.0, atol=1e-15)
    np.testing.assert_allclose(o["conf"], 0.5, atol=1e-15)
    np.testing.assert_allclose(o["bce"], np.log(2.0), atol=1e-12)
    assert abs(o["loss"] - (0.1 * np.log(V) + np.log(2.0))) < 1e-12


def test_block_loss_disjoint_supports():
    """Draft and target concentrated on different tokens: L1 = 1, c* = 0."""
    V = 20
    x = _bl_inputs(1, 2, V, 3, 2)
    U = np.zeros((1, 2, V), np.float32)
    t = np.zeros((1, 2, V), np.float32)
    U[0, :, 3] = 200.0
    t[0, :, 11] = 200.0
    x.update(U=U, t=t, W2=np.zeros((V, 2), np.float32), y=np.array([[3, 11]], np.int32))
    o = oracle.block_loss(**x)
    np.testing.assert_allclose(o["l1"], 1.0, atol=1e-12)
    assert abs(o["ce"][0, 0]) < 1e-12 and abs(o["ce"][0, 1] - 200.0) < 1e-9
    # with c* = 0 the BCE is -log(1 - conf)
    np.testing.assert_allclose(o["bce"], -np.log1p(-o["conf"]), rtol=1e-12)


def test_block_loss_uses_the_given_previous_token():
    """W1 = I and W2 = c I (r = V): the bias is c on the given previous token
    only, so with U = 0 and y = x, CE = log(V - 1 + e^c) - c; with y != x,
    CE = log(V - 1 + e^c)."""
    V, c = 12, 2.5
    x = _bl_inputs(2, 4, V, 3, V, seed=3)
    x.update(U=np.zeros((2, 4, V), np.float32), W1=np.eye(V, dtype=np.float32),
             W2=(c * np.eye(V)).astype(np.float32))
    xp = np.array([[1, 5, 5, 0], [11, 2, 7, 3]], np.int32)
    y = np.array([[1, 5, 6, 0], [10, 2, 7, 4]], np.int32)
    x.update(xp=xp, y=y)
    o = oracle.block_loss(**x)
    lse = np.log(V - 1 + np.exp(c))
    np.testing.assert_allclose(o["ce"], np.where(y == xp, lse - c, lse), rtol=1e-12)


def test_block_loss_l1_matches_accept_rate_oracle():
    """With W2 = 0 the draft logits are U, so 1 - L1 is the accept-rate
    oracle's c* of (U, t) row by row."""
    x = _bl_inputs(3, 4, 300, 6, 8, seed=9)
    x["W2"] = np.zeros_like(x["W2"])
    o = oracle.block_loss(**x)
    cs = oracle.accept_rate(x["U"].reshape(12, 300), x["t"].reshape(12, 300))
    np.testing.assert_allclose(1.0 - o["l1"].reshape(-1), cs, atol=1e-13)


def test_block_loss_bce_is_binary_entropy_at_calibration():
    """V = 2: p_d = (1/2, 1/2), p_t = (1/4, 3/4) give L1 = 1/4, c* = 3/4; with
    conf = sigmoid(log 3) = 3/4 the BCE is the binary entropy H(3/4), its
    minimum over conf."""
    x = _bl_inputs(1, 1, 2, 2, 1)
    x.update(U=np.zeros((1, 1, 2), np.float32), t=np.array([[[0.0, np.log(3.0)]]], np.float32),
             W2=np.zeros((2, 1), np.float32), w_conf=np.zeros(3, np.float32), b_conf=float(np.log(3.0)))
    o = oracle.block_loss(**x)
    assert abs(o["l1"][0, 0] - 0.25) < 1e-7
    Hb = -(0.75 * np.log(0.75) + 0.25 * np.log(0.25))
    assert abs(o["conf"][0, 0] - 0.75) < 1e-7 and abs(o["bce"][0, 0] - Hb) < 1e-6
    for b in (np.log(2.0), np.log(4.0)):  # any other confidence costs more
        x["b_conf"] = float(b)
        assert oracle.block_loss(**x)["bce"][0, 0] > Hb + 1e-3


def test_block_loss_confidence_head_sees_h_and_the_previous_embedding():
    V, H, r = 9, 4, 3
    x = _bl_inputs(1, 2, V, H, r, seed=5)
    w = np.zeros(H + r, np.float32)
    w[1], w[H + 2] = 0.5, -2.0
    x.update(w_conf=w, b_conf=0.25)
    o = oracle.block_loss(**x)
    z = 0.5 * x["h"][0, :, 1].astype(np.float64) - 2.0 * x["W1"][x["xp"][0], 2].astype(np.float64) + 0.25
    np.testing.assert_allclose(o["conf"][0], 1 / (1 + np.exp(-z)), rtol=1e-12)


def test_block_loss_position_weights_and_mask():
    """One unmasked position: each term is that position's value.  Positions
    k = 1 and 3 (1-based): weights 1 and exp(-(3-1)/4) ([W] 7.2).  Invalid
    tokens give NaN and drop out."""
    x = _bl_inputs(1, 4, 40, 3, 4, seed=2)
    o = oracle.block_loss(**x)
    m = np.zeros((1, 4), np.float32)
    m[0, 2] = 1.0
    one = oracle.block_loss(**x, mask=m)
    assert abs(one["L_ce"] - o["ce"][0, 2]) < 1e-12 and abs(one["L_l1"] - o["l1"][0, 2]) < 1e-12
    assert abs(one["L_conf"] - o["bce"][0, 2]) < 1e-12
    m = np.array([[1, 0, 1, 0]], np.float32)
    two = oracle.block_loss(**x, mask=m, a_ce=1.0, a_l1=0.0, a_conf=0.0)
    w3 = np.exp(-(3 - 1) / 4.0)
    assert abs(two["loss"] - (o["ce"][0, 0] + w3 * o["ce"][0, 2]) / (1 + w3)) < 1e-12
    x["y"][0, 1] = 40
    x["xp"][0, 3] = -1
    bad = oracle.block_loss(**x)
    assert np.isnan(bad["ce"][0, 1]) and np.isnan(bad["bce"][0, 3])
    w = np.exp(-np.array([0, 2]) / 4.0)
    assert abs(bad["L_l1"] - (w[0] * o["l1"][0, 0] + w[1] * o["l1"][0, 2]) / w.sum()) < 1e-12
    m0 = np.zeros((1, 4), np.float32)
    assert oracle.block_loss(**x, mask=m0)["loss"] == 0.0
