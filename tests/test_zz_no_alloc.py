"""dspark_head_sample_noalloc (the sampler on the library's static per-GPU
scratch array) against dspark_head_sample with a workspace of its own, on
calls in a row whose inputs shrink, so that each call finds the scratch as
the previous, larger one left it."""
import ctypes

import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import synth
from helpers import dev

pytestmark = pytest.mark.gpu


def _case(B, gamma, V, H, r, dtype, gumbel, seed, w_sd=0.02, U_sd=3.0):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=H, r=r, dtype=dtype, w_sd=w_sd, U_sd=U_sd, wc_sd=0.01,
                           gumbel=gumbel, seed=seed)
    w, x = synth.sampler_weights(s), synth.sampler_batch(s)
    return [dev(v) for v in (x["U"], x["h"], w["W1"], w["W2"], w["w_conf"])] + [0.0, dev(x["x0"]), dev(x["G"])]


def _same(a, b):
    for k in ("tokens", "conf", "survival"):
        x, y = a[k], b[k]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), k


def test_noalloc_matches_the_workspace_entry_point_on_shrinking_calls():
    cases = [
        (64, 7, 151936, 5120, 256, "bf16", True, 8101),   # batched Gumbel, the resident kernel
        (1, 7, 151936, 5120, 256, "bf16", False, 8102),   # single request, the persistent screen
        (1, 7, 151936, 5120, 256, "bf16", False, 8102),   # the same call again on the same scratch
        (4, 7, 4096, 256, 32, "f32", False, 8103),        # smaller still: the per-step kernels
    ]
    for B, gamma, V, H, r, dt, gumbel, seed in cases:
        args = _case(B, gamma, V, H, r, dt, gumbel, seed, w_sd=0.02 if dt == "bf16" else 0.05)
        ref = dh.head_sample(*args)
        got = dh.head_sample_noalloc(*args)
        _same(got, ref)
        assert torch.all(got["tokens"] >= 0)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    L = dh.lib()
    need = L.dspark_head_sample_workspace_size(4096, 16, 151936, 0, 256, 1)
    assert need > 4 << 20
    fake = 0x1000  # never dereferenced: the size check fails before any launch
    st = L.dspark_head_sample_noalloc(4096, 16, 151936, 0, 256, 1, fake, None, fake, fake, fake, 0.0, fake, None,
                                      None, fake, fake, fake, None, None, None)
    assert st == 4  # DSPARK_ERR_WORKSPACE
