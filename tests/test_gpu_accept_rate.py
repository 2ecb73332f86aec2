"""GPU parity of dspark_accept_rate against the CPU oracle (abs err <= 1e-4)."""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import oracle
import synth
from helpers import PROB_ATOL, dev, workspace_dirty_bytes

pytestmark = pytest.mark.gpu


def test_tiny_workload():
    d, t = synth.accept_inputs(synth.ACCEPT_TINY)
    got = dh.accept_rate(dev(d), dev(t)).cpu().numpy()
    assert np.abs(got - oracle.accept_rate(d, t)).max() <= PROB_ATOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,V,pad", [(1, 1, 0), (3, 2, 0), (5, 4099, 0), (7, 4099, 13), (4, 8192, 8),
                                     (2, 151936, 0), (9, 30001, 3)])
def test_shapes_and_strides(dtype, N, V, pad):
    s = synth.AcceptShape(N=N, V=V + pad, dtype=dtype, d_sd=3.0, scale=0.8, t_sd=1.5, seed=1234 + V + pad)
    d, t = synth.accept_inputs(s)
    got = dh.accept_rate(dev(d), dev(t), V=V).cpu().numpy()
    ref = oracle.accept_rate(d, t, V=V)
    assert np.abs(got - ref).max() <= PROB_ATOL


def test_identical_rows_give_exactly_one():
    d, _ = synth.accept_inputs(synth.AcceptShape(N=6, V=20000, dtype="bf16", d_sd=3, scale=1, t_sd=1, seed=5))
    got = dh.accept_rate(dev(d), dev(d.copy())).cpu().numpy()
    assert np.all(got == 1.0)


def test_different_row_strides():
    s = synth.AcceptShape(N=5, V=3000, dtype="f32", d_sd=2, scale=1.0, t_sd=0.5, seed=8)
    d, t = synth.accept_inputs(s)
    tp = np.zeros((5, 3072), np.float32)
    tp[:, :3000] = t
    got = dh.accept_rate(dev(d), dev(tp), V=3000).cpu().numpy()
    assert np.abs(got - oracle.accept_rate(d, t)).max() <= PROB_ATOL


def test_training_workload_sampled_rows():
    """N=2048 rows x V=151936 bf16 in one launch; the oracle checks 48 rows."""
    s = synth.ACCEPT_TRAIN
    d, t = synth.accept_inputs(s)
    out = torch.full((s.N,), float("nan"), dtype=torch.float32, device="cuda")  # an unwritten row stays NaN
    call, _ = dh.prepare_accept_rate(dev(d), dev(t), out=out)
    call()
    got = out.cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, s.N - 1], np.random.default_rng(3).integers(0, s.N, 45)]))
    ref = oracle.accept_rate(np.ascontiguousarray(d[rows]), np.ascontiguousarray(t[rows]))
    assert np.abs(got[rows] - ref).max() <= PROB_ATOL
    assert np.all(np.isfinite(got)) and np.all(got > -1e-6) and np.all(got < 1 + 1e-6)


def test_repeat_runs_are_bitwise_identical():
    d, t = synth.accept_inputs(synth.AcceptShape(N=64, V=151936, dtype="bf16", d_sd=3, scale=0.8, t_sd=1.5, seed=2))
    dd, tt = dev(d), dev(t)
    a = dh.accept_rate(dd, tt)
    b = dh.accept_rate(dd, tt)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_empty():
    z = torch.zeros((0, 10), device="cuda")
    assert dh.accept_rate(z, z).shape == (0,)


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves calls of different shapes in a row:
    every call leaves it zeroed, so results match fresh workspaces bitwise."""
    import draft_head_sampling_amd as dh_

    shapes = [(64, 151936, "bf16"), (5, 30001, "bf16"), (300, 8192, "f32"), (64, 151936, "bf16"), (1, 151936, "bf16")]
    big = max(dh_.lib().dspark_accept_rate_workspace_size(N, V, 1) for N, V, _ in shapes)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for i, (N, V, dt) in enumerate(shapes):
        d, t = synth.accept_inputs(synth.AcceptShape(N=N, V=V, dtype=dt, d_sd=3, scale=0.8, t_sd=1.5, seed=40 + i))
        dd, tt = dev(d), dev(t)
        a = dh.accept_rate(dd, tt, workspace=ws)
        b = dh.accept_rate(dd, tt)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (N, V)
    assert workspace_dirty_bytes(ws) == 0


def _nan_filled_call(d, t, ws):
    out = torch.full((d.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
    call, _ = dh.prepare_accept_rate(d, t, out=out, workspace=ws)
    call()
    return out


def test_whole_row_clusters_leave_the_row_counter_clear():
    """Regression: with rows short enough for one workgroup each (a cluster
    of one), rows after the first wave of clusters are still claimed from
    the workspace's row counter.  Every call must leave that counter at
    zero, or the next call on the same workspace skips rows.  More rows than
    fit on the GPU at once, twice on one workspace, then the training-width
    workload on the same workspace; every output starts as NaN."""
    import draft_head_sampling_amd as dh_

    small = synth.AcceptShape(N=4096, V=8192, dtype="f32", d_sd=3, scale=0.8, t_sd=1.5, seed=77)
    big = synth.ACCEPT_TRAIN
    nbytes = max(dh_.lib().dspark_accept_rate_workspace_size(small.N, small.V, 0),
                 dh_.lib().dspark_accept_rate_workspace_size(big.N, big.V, 1))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    d, t = synth.accept_inputs(small)
    ref = oracle.accept_rate(d, t)
    dd, tt = dev(d), dev(t)
    for _ in range(2):
        got = _nan_filled_call(dd, tt, ws).cpu().numpy()
        assert np.all(np.isfinite(got))
        assert np.abs(got - ref).max() <= PROB_ATOL
        assert workspace_dirty_bytes(ws) == 0
    del dd, tt
    d, t = synth.accept_inputs(big)
    dd, tt = dev(d), dev(t)
    got = _nan_filled_call(dd, tt, ws)
    fresh = _nan_filled_call(dd, tt, None)
    assert torch.equal(got.view(torch.int32), fresh.view(torch.int32))
    g = got.cpu().numpy()
    assert np.all(np.isfinite(g))
    rows = np.array([0, 1, 777, big.N - 1])
    ref = oracle.accept_rate(np.ascontiguousarray(d[rows]), np.ascontiguousarray(t[rows]))
    assert np.abs(g[rows] - ref).max() <= PROB_ATOL
    assert workspace_dirty_bytes(ws) == 0
