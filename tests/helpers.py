"""Shared helpers for the GPU parity tests: host<->device marshalling and the
comparison rules.

Comparison rules (the tolerances the workloads are graded on):
  tokens, sort order, prefix lengths      bit-exact
  logits and Markov bias                  normwise relative error <= 2e-3 per
                                          (request, position) row:
                                          max|gpu - ref| / max|ref|
  confidence, survival, accept rate       absolute error <= 1e-4
Near-ties: where the oracle's top-1/top-2 score margin is below 1e-3 the two
sides may legitimately pick different tokens (binary32 rounding of the score
differs with accumulation order); the comparison then teacher-forces both on
the oracle's token and continues.
"""
from __future__ import annotations

import numpy as np
import torch

import draft_head_sampling_amd as dh
import oracle

TIE_MARGIN = 1e-3
LOGIT_RTOL = 2e-3
PROB_ATOL = 1e-4


def dev(a: np.ndarray | None, device="cuda"):
    """numpy -> CUDA tensor; uint16 arrays are bfloat16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def workspace_dirty_bytes(ws: torch.Tensor) -> int:
    """Non-zero bytes of a workspace after a call, not counting the header's
    path-flags word (bytes 12-15), which kernels only OR into and no kernel
    reads.  A call that completes leaves every other byte zero."""
    b = ws.view(torch.uint8).clone()
    b[12:16] = 0
    return int(b.count_nonzero())


def normwise_rel(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max|gpu - ref| / max|ref| (rows = last axis)."""
    num = np.abs(gpu.astype(np.float64) - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def run_gpu_sampler(x: dict, w: dict, force: np.ndarray | None, want_logits: bool, device="cuda", workspace=None):
    out = dh.head_sample(dev(x["U"], device), dev(x["h"], device), dev(w["W1"], device), dev(w["W2"], device),
                         dev(w["w_conf"], device), w["b_conf"], dev(x["x0"], device), dev(x.get("G"), device),
                         dev(force, device), want_logits=want_logits, Wg=dev(w.get("Wg"), device),
                         Wr=None if w.get("Wr") is None else tuple(dev(a, device) for a in w["Wr"]),
                         workspace=workspace)
    return {k: v.cpu().numpy() for k, v in out.items()}


def sampler_parity(x: dict, w: dict, want_logits: bool = False, device="cuda", workspace=None):
    """Compare the HIP sampler with the oracle under the near-tie protocol.

    At the first unexplained token mismatch of a request the oracle's margin
    must be below TIE_MARGIN; that position is then accepted as a tie, both
    sides are teacher-forced on the oracle's tokens up to it, and the
    comparison reruns.  At accepted ties the GPU's token must score within
    TIE_MARGIN of the oracle's best score.

    Returns (gpu outputs, oracle outputs, number of accepted ties)."""
    B, gamma, _ = x["U"].shape
    force = np.full((B, gamma), -1, np.int32)
    tie = np.zeros((B, gamma), bool)
    for _ in range(B * gamma + 1):
        f = force if tie.any() else None
        ref = oracle.head_sample(x["U"], x["h"], w["W1"], w["W2"], w["w_conf"], w["b_conf"], x["x0"], x.get("G"),
                                 f, want_logits=want_logits or tie.any(), Wg=w.get("Wg"), Wr=w.get("Wr"))
        got = run_gpu_sampler(x, w, f, want_logits, device, workspace)
        mism = (got["tokens"] != ref["tokens"]) & ~tie
        if not mism.any():
            break
        for b in np.unique(np.argwhere(mism)[:, 0]):
            k = int(np.argmax(mism[b]))
            assert ref["margin"][b, k] < TIE_MARGIN, (
                f"token mismatch at request {b} step {k}: gpu {got['tokens'][b, k]} oracle {ref['tokens'][b, k]}"
                f" (oracle margin {ref['margin'][b, k]:.3g} >= {TIE_MARGIN})")
            tie[b, k] = True
            force[b, : k + 1] = ref["tokens"][b, : k + 1]
    else:
        raise AssertionError("tokens still differ after teacher forcing")
    if tie.any():
        score = ref["logits"] + (x["G"].astype(np.float64) if x.get("G") is not None else 0.0)
        for b, k in np.argwhere(tie):
            g = got["tokens"][b, k]
            assert 0 <= g < score.shape[2] and score[b, k, g] >= score[b, k].max() - TIE_MARGIN
    np.testing.assert_array_equal(got["tokens"][~tie], ref["tokens"][~tie])
    assert np.abs(got["conf"] - ref["conf"]).max() <= PROB_ATOL
    assert np.abs(got["survival"] - ref["survival"]).max() <= PROB_ATOL
    if want_logits:
        assert normwise_rel(got["logits"], ref["logits"]) <= LOGIT_RTOL
        assert normwise_rel(got["bias"], ref["bias"]) <= LOGIT_RTOL
    return got, ref, int(tie.sum())
