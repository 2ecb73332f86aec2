"""The weights-only W2 bound of the single-request screen
(dspark_w2_bound) and the sampler call that uses it
(dspark_head_sample_w2bound, DSpark's sampling loop: a step's winner is
proved from U and a bound on the Markov bias, which needs the largest W2
row norm).  The bound's words against an fp64 reading of W2; the bounded
call against the plain call and the oracle; the fingerprint's verification
when W2 moves or changes in place."""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import synth
from helpers import dev, sampler_parity, workspace_dirty_bytes

pytestmark = pytest.mark.gpu

TAG = 0x5B0D2A7E


def _sqnorms(W2_bits):
    W = synth.bf16_to_f32(W2_bits).astype(np.float64)
    return (W * W).sum(axis=1)


def _f32(word):
    return float(np.array([word], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("V", [151936, 70001, 64, 1])
def test_bound_words(V):
    rng = np.random.default_rng(V)
    W2 = synth.f32_to_bf16(rng.normal(0, 0.05, (V, 256)).astype(np.float32))
    W2[V // 3] = synth.f32_to_bf16(np.full(256, 0.5, np.float32))  # one large row (squared norm 64)
    t = dev(W2)
    b = dh.w2_bound(t).cpu().numpy().view(np.uint32)
    n2 = _sqnorms(W2)
    sample = np.arange(64) * (V // 64)  # the rows the screen samples
    # binary32 sums of 256 exact bf16 squares: a few ulp
    assert abs(_f32(b[0]) - n2.max()) <= 3e-5 * n2.max()
    assert abs(_f32(b[1]) - n2[sample].max()) <= 3e-5 * n2[sample].max()
    assert b[2] == V and b[3] == 0 and b[4] == 256
    addr = t.data_ptr()
    assert b[5] == addr & 0xFFFFFFFF and b[6] == addr >> 32
    assert b[7] == TAG


def _gpu(x, w, W2t, bound=None, ws=None):
    G = dev(x["G"]) if x.get("G") is not None else None
    call, out = dh.prepare_head_sample(dev(x["U"]), dev(x["h"]), dev(w["W1"]), W2t, dev(w["w_conf"]), w["b_conf"],
                                       dev(x["x0"]), G, workspace=ws, w2_bound=bound)
    call()
    torch.cuda.synchronize()
    return {k: out[k].cpu().numpy() for k in ("tokens", "conf", "survival")}


def _same(a, b, exact):
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    for k in ("conf", "survival"):
        if exact:
            np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32))
        else:
            np.testing.assert_allclose(a[k], b[k], rtol=0, atol=1e-6)


def _ws(s):
    return torch.zeros(dh.head_sample_workspace_size(1, s.gamma, s.V, s.H, s.r), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("kind", ["weak", "gumbel", "strong"])
def test_bounded_call_matches_the_streaming_call(kind):
    """The bench's workload (weak bias: every step on the screen), with Gumbel
    noise, and with a strong bias (the screen gives most steps to the
    exchange): the same tokens as dspark_head_sample, path flag 16, a clean
    workspace; and the oracle's tokens for one anchor."""
    b1 = synth.SAMPLER_B1
    s = b1 if kind != "gumbel" else synth.SamplerShape(
        B=1, gamma=b1.gamma, V=b1.V, H=b1.H, r=b1.r, dtype=b1.dtype, w_sd=b1.w_sd, U_sd=b1.U_sd, wc_sd=b1.wc_sd,
        gumbel=True, seed=b1.seed + 77)
    w = synth.sampler_weights(s, w_sd=0.5) if kind == "strong" else synth.sampler_weights(s)
    W2t = dev(w["W2"])
    bound = dh.w2_bound(W2t)
    ws = _ws(s)
    for anchor in (20, 21):
        x = synth.sampler_batch(s, batch_id=anchor)
        a = _gpu(x, w, W2t, None, ws)
        st0, p0 = dh.workspace_status(ws)
        b = _gpu(x, w, W2t, bound, ws)
        st1, p1 = dh.workspace_status(ws)
        assert st0 == 0 and st1 == 0
        assert p1 & dh.PATH_B1_BOUND and not p1 & dh.PATH_B1_BOUND_STALE, p1
        assert not p0 & (dh.PATH_B1_BOUND | dh.PATH_B1_BOUND_STALE), p0
        # same steps on the screen (no exchange on either side): same bits
        _same(a, b, exact=not ((p0 | p1) & dh.PATH_B1_EXCHANGE))
    assert workspace_dirty_bytes(ws) == 0
    got, ref, _ = sampler_parity(synth.sampler_batch(s, batch_id=20), w)  # the plain call against the oracle
    np.testing.assert_array_equal(got["tokens"], _gpu(synth.sampler_batch(s, batch_id=20), w, W2t, bound)["tokens"])


def test_stale_bound_is_not_trusted():
    """(a) The same weights at another address: the fingerprint names another
    W2, so the call streams W2 as dspark_head_sample does (same bits, no
    bound flag).  (b) W2 changed in place at a row the screen samples: the
    sampled norm no longer matches, so the call proves nothing from the bound
    and settles the block with the exchange (flags 32 and 2); its tokens are
    the oracle's for the changed weights."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s)
    W2t = dev(w["W2"])
    bound = dh.w2_bound(W2t)
    x = synth.sampler_batch(s, batch_id=3)
    ws = _ws(s)

    W2b = W2t.clone()
    a = _gpu(x, w, W2b, None, ws)
    dh.workspace_status(ws)
    b = _gpu(x, w, W2b, bound, ws)
    st, p = dh.workspace_status(ws)
    assert st == 0 and not p & (dh.PATH_B1_BOUND | dh.PATH_B1_BOUND_STALE), p
    _same(a, b, exact=True)

    W2f = synth.bf16_to_f32(w["W2"])
    W2f[0] *= 3.0  # row 0 is the first sampled row
    w_mod = dict(w, W2=synth.f32_to_bf16(W2f))
    W2t.copy_(dev(w_mod["W2"]))  # same address, new contents
    a = _gpu(x, w_mod, W2t, None, ws)
    dh.workspace_status(ws)
    b = _gpu(x, w_mod, W2t, bound, ws)
    st, p = dh.workspace_status(ws)
    assert st == 0 and p & dh.PATH_B1_BOUND_STALE and p & dh.PATH_B1_EXCHANGE, p
    _same(a, b, exact=False)
    assert workspace_dirty_bytes(ws) == 0
    got, ref, _ = sampler_parity(x, w_mod)
    np.testing.assert_array_equal(got["tokens"], b["tokens"])
