"""Give-ups of the waits between workgroups, and the path flags, as seen at
the C ABI (dspark_workspace_status, dspark_set_wait_limit).

The failure path is forced from the host: a wait limit of 0 polls makes every
wait for another workgroup give up at once, so every kernel still runs to
completion -- no workgroup is held back and nothing hangs.  Each case checks
that the give-up is reported, that the outputs are the documented -1 / NaN,
and that a zero-filled workspace then serves a normal call again.
"""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import synth
from helpers import dev, workspace_dirty_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture
def no_waits():
    prev = dh.set_wait_limit(0)
    try:
        yield
    finally:
        dh.set_wait_limit(prev)


def _sampler_case(B, gamma, V, gumbel, seed):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=64, r=256, dtype="bf16", w_sd=0.05, U_sd=2.0, wc_sd=0.05,
                           gumbel=gumbel, seed=seed)
    w, x = synth.sampler_weights(s), synth.sampler_batch(s)
    args = [dev(v) for v in (x["U"], x["h"], w["W1"], w["W2"], w["w_conf"])] + [0.1, dev(x["x0"]), dev(x["G"])]
    return s, args


def _fresh_then_give_up_then_recover(s, args, expect_paths, ws_bytes=None, **head):
    if ws_bytes is None:
        ws_bytes = dh.head_sample_workspace_size(s.B, s.gamma, s.V, 64, 256)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    good = dh.head_sample(*args, **head)  # a workspace of its own
    prev = dh.set_wait_limit(0)
    try:
        bad = dh.head_sample(*args, workspace=ws, **head)
        st, paths = dh.workspace_status(ws)
    finally:
        dh.set_wait_limit(prev)
    assert st == 1
    assert paths & expect_paths == expect_paths
    assert torch.all(bad["tokens"] == -1)
    assert torch.all(torch.isnan(bad["conf"])) and torch.all(torch.isnan(bad["survival"]))
    ws.zero_()  # the documented recovery
    again = dh.head_sample(*args, workspace=ws, **head)
    assert dh.workspace_status(ws)[0] == 0
    for k in good:
        assert torch.equal(good[k].view(torch.int32) if good[k].dtype == torch.float32 else good[k],
                           again[k].view(torch.int32) if again[k].dtype == torch.float32 else again[k]), k
    assert workspace_dirty_bytes(ws) == 0


def test_single_request_screen_gives_up():
    """B=1, bf16, rank 256, gamma <= 8: the persistent kernel's candidate
    screen (its coordinator never sees the lists)."""
    s, args = _sampler_case(1, 7, 70001, False, 901)
    _fresh_then_give_up_then_recover(s, args, 0)


def test_single_request_exchange_gives_up():
    """B=1 with gamma = 9: the persistent kernel's grid-wide per-step
    exchange from the first step on."""
    s, args = _sampler_case(1, 9, 70001, True, 902)
    _fresh_then_give_up_then_recover(s, args, dh.PATH_B1_EXCHANGE)


def test_batched_resident_gives_up():
    """B=64, bf16, rank 256: the resident-W2 kernel's per-step exchange."""
    s, args = _sampler_case(64, 4, 20000, True, 903)
    _fresh_then_give_up_then_recover(s, args, dh.PATH_RESIDENT)


@pytest.mark.parametrize("head", ["gated", "rnn"])
def test_batched_resident_gated_and_rnn_heads_give_up(head):
    """B=64, bf16, rank 256 with a gated or RNN head: the resident kernel's
    exchange of the head's embedding columns gives up too."""
    s, args = _sampler_case(64, 3, 20000, True, 905)
    if head == "gated":
        extra = {"Wg": dev(synth.gate_weights(s, 0.05))}
        n = dh.lib().dspark_head_sample_gated_workspace_size(64, 3, 20000, 64, 256, 1)
    else:
        extra = {"Wr": tuple(dev(a) for a in synth.rnn_weights(s, 0.05))}
        n = dh.lib().dspark_head_sample_rnn_workspace_size(64, 3, 20000, 64, 256, 1)
    paths = dh.PATH_RESIDENT if torch.cuda.get_device_properties(0).multi_processor_count >= 256 else 0
    _fresh_then_give_up_then_recover(s, args, paths, ws_bytes=n, **extra)


def test_accept_rate_cluster_gives_up(no_waits):
    d, t = synth.accept_inputs(synth.AcceptShape(N=64, V=151936, dtype="bf16", d_sd=3, scale=0.8, t_sd=1.5, seed=904))
    dd, tt = dev(d), dev(t)
    ws = torch.zeros(dh.lib().dspark_accept_rate_workspace_size(64, 151936, 1), dtype=torch.uint8, device="cuda")
    bad = dh.accept_rate(dd, tt, workspace=ws)
    st, paths = dh.workspace_status(ws)
    assert st == 1 and paths & dh.PATH_ACCEPT_CLUSTER
    assert torch.all(torch.isnan(bad))
    dh.set_wait_limit(-1)
    ws.zero_()
    good = dh.accept_rate(dd, tt, workspace=ws)
    assert dh.workspace_status(ws)[0] == 0
    assert torch.equal(good.view(torch.int32), dh.accept_rate(dd, tt).view(torch.int32))
    assert torch.all(torch.isfinite(good))
    assert workspace_dirty_bytes(ws) == 0


def test_verify_draw_gives_up(no_waits):
    vi = synth.verify_inputs(synth.VERIFY_TINY)
    args = [dev(vi[k]) for k in ("d", "t", "x", "u", "G")]
    ws = torch.zeros(dh.lib().dspark_verify_workspace_size(4, 7, 4096, 0), dtype=torch.uint8, device="cuda")
    bad = dh.verify(*args, workspace=ws)
    assert dh.workspace_status(ws)[0] == 1
    assert torch.all(bad["next_token"] == -1)
    dh.set_wait_limit(-1)
    ws.zero_()
    good = dh.verify(*args, workspace=ws)
    ref = dh.verify(*args)
    assert dh.workspace_status(ws)[0] == 0
    assert torch.equal(good["next_token"], ref["next_token"]) and torch.all(good["next_token"] >= 0)
    assert torch.equal(good["n_accepted"], ref["n_accepted"])
    assert workspace_dirty_bytes(ws) == 0


def test_debug_mode_raises_on_a_give_up(monkeypatch, no_waits):
    """DSPARK_DEBUG=1: the binding synchronises after the call and raises."""
    monkeypatch.setenv("DSPARK_DEBUG", "1")
    s, args = _sampler_case(1, 5, 5000, False, 905)
    with pytest.raises(dh.DsparkGaveUp):
        dh.head_sample(*args)
    dh.set_wait_limit(-1)
    out = dh.head_sample(*args)  # a fresh zero-filled workspace, default limit: no error
    assert torch.all(out["tokens"] >= 0)


def test_wait_limit_is_checked_on_the_host():
    with pytest.raises(dh.DsparkError):
        dh.set_wait_limit(2**31)
    prev = dh.set_wait_limit(-5)
    assert dh.set_wait_limit(prev) == -1
