"""GPU parity of dspark_verify (rejection-sampling verification) against the
CPU oracle.

Accept decisions and the number of kept tokens are compared exactly.  The
decision u < min(1, p_t/p_d) is taken in binary32 on the GPU and in binary64
by the oracle, so the uniforms are first moved away from the oracle's
thresholds (to at least 2e-4 on the same side; DECISION_GAP), which keeps
every decision and makes the comparison well-posed.  The drawn token is an
argmax: exact unless the oracle's top-1/top-2 margin is below 1e-3, where the
GPU's token must score within 1e-3 of the best.  accept_prob: abs err <= 1e-4.
"""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import oracle
import synth
from helpers import PROB_ATOL, TIE_MARGIN, dev, workspace_dirty_bytes

pytestmark = pytest.mark.gpu

DECISION_GAP = 2e-4


def _widen(a):
    return synth.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _softmax64(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _separate_decisions(inp, n_draft=None):
    """Move each uniform the oracle compares away from its threshold, keeping
    the side it is on, so that binary32 and binary64 take the same decision."""
    ref = oracle.verify(inp["d"], inp["t"], inp["x"], inp["u"], inp["G"], n_draft)
    a = ref["accept_prob"]
    u = inp["u"].astype(np.float64)
    near = np.isfinite(a) & (a < 1.0) & (np.abs(u - a) < DECISION_GAP)
    u = np.where(near, np.where(u < a, a - DECISION_GAP, a + DECISION_GAP), u)
    out = dict(inp)
    out["u"] = np.clip(u, 0.0, 1.0 - 2**-24).astype(np.float32)
    return out


def _score(inp, b, pos, residual, v):
    """fp64 score of token v in request b's draw."""
    t = _widen(inp["t"][b, pos])
    g = inp["G"][b].astype(np.float64)
    if residual:
        r = _softmax64(t) - _softmax64(_widen(inp["d"][b, pos]))
        return np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)[v] + g[v]
    return t[v] + g[v]


def verify_parity(inp, n_draft=None, device="cuda"):
    inp = _separate_decisions(inp, n_draft)
    ref = oracle.verify(inp["d"], inp["t"], inp["x"], inp["u"], inp["G"], n_draft)
    got = dh.verify(dev(inp["d"], device), dev(inp["t"], device), dev(inp["x"], device), dev(inp["u"], device),
                    dev(inp["G"], device), dev(n_draft, device), want_accept_prob=True)
    got = {k: v.cpu().numpy() for k, v in got.items()}
    np.testing.assert_array_equal(got["n_accepted"], ref["n_acc"])
    a_ref, a_got = ref["accept_prob"], got["accept_prob"]
    assert np.array_equal(np.isnan(a_ref), np.isnan(a_got))
    fin = np.isfinite(a_ref)
    assert np.abs(a_got[fin] - a_ref[fin]).max(initial=0.0) <= PROB_ATOL
    ties = 0
    for b in range(len(ref["n_acc"])):
        g, r = int(got["next_token"][b]), int(ref["next_token"][b])
        if g == r:
            continue
        assert ref["margin"][b] < TIE_MARGIN, f"request {b}: gpu {g} oracle {r} margin {ref['margin'][b]:.3g}"
        pos, res = int(ref["sample_pos"][b]), bool(ref["residual"][b])
        assert 0 <= g < inp["t"].shape[2]
        assert _score(inp, b, pos, res, g) >= _score(inp, b, pos, res, r) - TIE_MARGIN
        ties += 1
    return got, ref, ties


def test_tiny_workload():
    got, ref, ties = verify_parity(synth.verify_inputs(synth.VERIFY_TINY))
    assert ties == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,gamma,V", [(1, 1, 1), (3, 2, 2), (5, 4, 777), (4, 7, 4099), (6, 3, 8192),
                                       (2, 16, 30001), (17, 1, 1000)])
def test_shapes(dtype, B, gamma, V):
    s = synth.VerifyShape(B=B, gamma=gamma, V=V, dtype=dtype, d_sd=2.0, scale=0.9, t_sd=0.7, seed=77 + V + gamma)
    verify_parity(synth.verify_inputs(s))


def test_draft_counts_invalid_tokens_and_identical_distributions():
    s = synth.VerifyShape(B=8, gamma=5, V=5000, dtype="bf16", d_sd=2.0, scale=0.9, t_sd=0.7, seed=501)
    inp = synth.verify_inputs(s)
    inp["x"][1, 0] = -1
    inp["x"][2, 3] = 5000
    inp["d"][3] = inp["t"][3, :5]  # identical: every drafted token is kept
    inp["d"][4, 1] = inp["t"][4, 1]
    inp["x"][4, 1] = 5000 + 7      # invalid where d == t: an empty residual, the p_t draw
    n = np.array([5, 5, 5, 5, 5, 0, -3, 99], np.int32)  # 0, clamped to 0, clamped to 5
    got, ref, _ = verify_parity(inp, n)
    assert got["n_accepted"][1] == 0 and got["n_accepted"][3] == 5 and got["n_accepted"][5] == 0


def test_zero_requests_and_zero_gamma():
    s = synth.VerifyShape(B=3, gamma=0, V=300, dtype="f32", d_sd=2.0, scale=0.9, t_sd=0.7, seed=9)
    inp = synth.verify_inputs(s)
    got, ref, _ = verify_parity(inp)
    assert np.all(got["n_accepted"] == 0)
    assert np.array_equal(got["next_token"], np.argmax(inp["t"][:, 0] + inp["G"], axis=1))
    z = torch.zeros((0, 2, 10), device="cuda")
    out = dh.verify(z[:, :1], z, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                    torch.zeros((0, 1), device="cuda"), torch.zeros((0, 10), device="cuda"))
    assert out["n_accepted"].shape == (0,)


def test_batched_serving_workload_full_size():
    """B=64, gamma=7, V=151936 bf16 in the launch configuration the benchmark
    times; the oracle checks every request."""
    got, ref, ties = verify_parity(synth.verify_inputs(synth.VERIFY_B64))
    assert ties <= 2


def test_repeat_runs_are_bitwise_identical_and_workspace_is_left_zero():
    inp = synth.verify_inputs(synth.VERIFY_B64, B=16)
    args = [dev(inp[k]) for k in ("d", "t", "x", "u", "G")]
    B, gamma = inp["x"].shape
    ws = torch.zeros(dh.lib().dspark_verify_workspace_size(64, 16, 151936, 1), dtype=torch.uint8, device="cuda")
    a = dh.verify(*args, want_accept_prob=True, workspace=ws)
    assert workspace_dirty_bytes(ws) == 0
    b = dh.verify(*args, want_accept_prob=True, workspace=ws)
    for k in ("n_accepted", "next_token"):
        assert torch.equal(a[k], b[k])
    assert torch.equal(a["accept_prob"].view(torch.int32), b["accept_prob"].view(torch.int32))
    # a smaller shape through the same workspace
    small = synth.verify_inputs(synth.VerifyShape(B=3, gamma=2, V=999, dtype="f32", d_sd=2.0, scale=0.9, t_sd=0.7,
                                                  seed=3))
    c = dh.verify(*[dev(small[k]) for k in ("d", "t", "x", "u", "G")], workspace=ws)
    d = dh.verify(*[dev(small[k]) for k in ("d", "t", "x", "u", "G")])
    assert torch.equal(c["next_token"], d["next_token"]) and torch.equal(c["n_accepted"], d["n_accepted"])
    assert workspace_dirty_bytes(ws) == 0
