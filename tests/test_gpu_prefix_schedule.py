"""GPU parity of dspark_prefix_schedule against the CPU oracle: prefix
lengths, sorted order, survivals, Theta and the selection count bit-exact."""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import oracle
import synth
from helpers import dev

pytestmark = pytest.mark.gpu


def _check(conf, sps):
    conf = np.ascontiguousarray(conf, np.float32)
    sps = np.ascontiguousarray(sps, np.float64)
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in dh.prefix_schedule(dev(conf), dev(sps)).items()}
    r = oracle.prefix_schedule(conf, sps)
    np.testing.assert_array_equal(g["prefix_len"], r["prefix_len"])
    np.testing.assert_array_equal(g["order"], r["order"])
    np.testing.assert_array_equal(g["survival"].view(np.uint32), r["survival"].view(np.uint32))
    assert g["n_selected"][0] == r["n_selected"]
    assert g["theta"][0] == r["theta"], (g["theta"][0], r["theta"])
    return r


def test_training_workload_stated_curve():
    s = synth.SCHEDULE_TRAIN
    r = _check(synth.schedule_conf(s), synth.sps_table(s.n_sps, "tokens"))
    assert r["n_selected"] == s.n_sps - s.B  # increasing curve: stops at the table's end


def test_training_workload_step_rate_curve():
    s = synth.SCHEDULE_TRAIN
    r = _check(synth.schedule_conf(s), synth.sps_table(s.n_sps, "steps"))
    assert 0 < r["n_selected"] < s.B * s.gamma


@pytest.mark.parametrize("seed", range(12))
def test_random_small(seed):
    rng = np.random.default_rng(seed)
    B, gamma = int(rng.integers(1, 40)), int(rng.integers(1, 20))
    conf = (1 / (1 + np.exp(-rng.normal(1.0, 2.0, (B, gamma))))).astype(np.float32)
    n_sps = B + int(rng.integers(0, B * gamma + 5))
    kind = seed % 3
    n = np.arange(1, n_sps + 1, dtype=np.float64)
    sps = {0: 1.0 / (rng.uniform(0.5, 3) + rng.uniform(0.001, 0.5) * n), 1: n / (2.0 + 0.004 * n),
           2: np.where(n <= n_sps // 2, 1.0, 0.6) * n / (1 + 0.01 * n)}[kind]
    _check(conf, sps)


def test_ties_zeros_ones_and_empty_block():
    _check(np.full((5, 3), 0.5), np.ones(40))
    conf = np.array([[1.0, 1.0, 0.0], [0.0, 1.0, 1.0], [1.0, 0.5, 0.25]], np.float32)
    _check(conf, synth.sps_table(12, "tokens"))
    _check(conf, synth.sps_table(12, "steps"))
    _check(np.zeros((4, 0), np.float32), synth.sps_table(8, "steps"))
    _check(np.full((3, 2), 0.5), np.array([1.0, 1.0, 3.0, 0.1, 0.1, 0.1, 0.1, 0.1]))  # first pair lowers Theta


def test_tiny_survivals_past_the_exact_run():
    # survivals far below 2^-17 under an increasing curve: the scan runs past
    # the exactly-summable run (the rounded increments of the tail)
    rng = np.random.default_rng(5)
    conf = rng.uniform(1e-4, 0.05, (64, 16)).astype(np.float32)
    conf[:, 0] = rng.uniform(0.5, 1.0, 64).astype(np.float32)
    r = _check(conf, synth.sps_table(64 * 17, "tokens"))
    assert r["n_selected"] == 64 * 16


def test_largest_supported_pair_count():
    rng = np.random.default_rng(6)
    conf = (1 / (1 + np.exp(-rng.normal(1.5, 1.5, (512, 16))))).astype(np.float32)
    _check(conf, synth.sps_table(9000, "steps"))
    _check(conf, synth.sps_table(9000, "tokens"))


def test_single_request():
    _check(np.array([[0.9, 0.8, 0.7, 0.2]], np.float32), synth.sps_table(5, "steps"))
    _check(np.array([[0.9, 0.8, 0.7, 0.2]], np.float32), np.array([1.0]))


def test_tail_ties_and_binade_crossings_finish_in_order():
    """Past the exactly-summable run the kernel sums rounded increments in
    parallel; an increment exactly half-way between two binary64 steps (a
    tie) or a running sum that crosses a power of two makes it finish pair by
    pair instead.  Both must give the sequential scan's result bit for bit."""
    tie = np.float32(1.5 * 2.0**-50)  # half-way between multiples of 2^-50 (tau in [4, 8))
    conf = np.array([[0.9, 0.8], [0.7, 0.5], [tie, 0.5], [np.float32(3 * 2.0**-52), 1.0]], np.float32)
    _check(conf, synth.sps_table(16, "tokens"))
    # one request: tau = 2 - 2^-20 after the first pair, then 63 survivals of
    # about 2^-24 carry it past 2 (the binade of the running sum changes)
    conf = np.ones((1, 64), np.float32)
    conf[0, 0] = np.float32(1 - 2.0**-20)
    conf[0, 1] = np.float32(2.0**-24)
    r = _check(conf, synth.sps_table(80, "tokens"))
    assert r["n_selected"] == 64


@pytest.mark.parametrize("B,gamma,seed", [(300, 9, 11), (257, 16, 12), (1000, 7, 13), (8192, 1, 14), (2, 4096, 15),
                                          (3, 2730, 16), (1, 8192, 17), (640, 12, 18)])
def test_many_workgroup_tiles_and_ragged_pair_counts(B, gamma, seed):
    """Pair counts that span several 1024-pair slices with a ragged last one,
    odd and even request counts (the transposed key layout pads the request
    stride only when it fits), one request or one position per request, and
    survivals rounded to eighths so that many pairs tie."""
    rng = np.random.default_rng(seed)
    conf = (1 / (1 + np.exp(-rng.normal(1.5, 1.5, (B, gamma))))).astype(np.float32)
    if seed % 2 == 0:
        conf = (np.round(conf * 8) / 8).astype(np.float32)
    n = B * gamma
    _check(conf, synth.sps_table(B + n, "steps"))
    _check(conf, synth.sps_table(B + n // 2 + 1, "tokens"))


def test_signed_zero_confidences_tie_with_zero():
    """-0 is a confidence in [0, 1] equal to 0: its pairs tie with those of
    +0 survivals and keep request and position order; the survival written
    out keeps the product's sign."""
    conf = np.array([[-0.0, -0.0, 0.5], [0.0, 0.5, 1.0], [0.3, -0.0, 1.0], [0.9, 0.0, -0.0]], np.float32)
    for k in (4, 8, 16):
        _check(conf, synth.sps_table(k, "tokens"))
        _check(conf, np.ones(k))


@pytest.mark.parametrize("tie_share,seed", [(0.02, 21), (0.2, 22)])
def test_tail_ties_spread_over_many_waves(tie_share, seed):
    """Past the exact run the kernel sums rounded increments in parallel and
    settles ties (a survival exactly half-way between two binary64 steps of
    the running sum) from the parity of the sum before each one.  Here the
    exact run is 512 survivals of 0.5 (tau = 768 after it, so one step is
    2^-43) and the tail holds 7680 pairs over fifteen waves, some requests'
    second survival a tie (2k+1) 2^-44: the parity must carry across waves
    with and without ties (13 and 111 ties here, in waves 1-5 and 1-9).
    """
    rng = np.random.default_rng(seed)
    B, g = 512, 16
    conf = np.empty((B, g), np.float32)
    conf[:, 0] = 0.5
    c = np.exp2(rng.uniform(-42, -30, B)).astype(np.float32)  # many bits below one step: hardly ever a tie
    tie = rng.random(B) < tie_share
    k = rng.integers(1, 2**10, B)
    c[tie] = ((2 * k[tie] + 1) * 2.0**-43).astype(np.float32)
    conf[:, 1] = c
    conf[:, 2:] = rng.uniform(0.5, 1.0, (B, g - 2)).astype(np.float32)
    r = _check(conf, synth.sps_table(B + B * g, "tokens"))
    assert r["n_selected"] == B * g


@pytest.mark.parametrize("B,gamma", [(256, 16), (300, 9), (3, 5)])
def test_confidences_not_16_byte_aligned(B, gamma):
    """The confidences read with 16-byte loads only from a 16-byte aligned
    array; a view four bytes into a buffer takes the element-wise path."""
    rng = np.random.default_rng(B * 31 + gamma)
    conf = (1 / (1 + np.exp(-rng.normal(1.5, 1.5, (B, gamma))))).astype(np.float32)
    sps = synth.sps_table(B + B * gamma, "steps")
    buf = torch.empty(B * gamma + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev(conf.ravel())
    view = buf[1:].view(B, gamma)
    assert view.data_ptr() % 16 != 0
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in dh.prefix_schedule(view, dev(sps)).items()}
    r = oracle.prefix_schedule(conf, sps)
    np.testing.assert_array_equal(g["prefix_len"], r["prefix_len"])
    np.testing.assert_array_equal(g["order"], r["order"])
    np.testing.assert_array_equal(g["survival"].view(np.uint32), r["survival"].view(np.uint32))
    assert g["n_selected"][0] == r["n_selected"]
    assert g["theta"][0] == r["theta"]
