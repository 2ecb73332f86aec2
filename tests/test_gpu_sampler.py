"""GPU parity of dspark_head_sample against the CPU oracle.

Workloads: the tiny fp32 sampler (B=4, gamma=7, V=4096, H=256, r=32), the
full-vocabulary single request (B=1, V=151936, H=5120, r=256, bf16, greedy)
and the batched Gumbel-max sampler (B=64, same shapes) in the launch
configuration the benchmark times; plus ragged and degenerate shapes.
"""
import numpy as np
import pytest
import torch

import draft_head_sampling_amd as dh
import oracle
import synth
from helpers import dev, run_gpu_sampler, sampler_parity, workspace_dirty_bytes

pytestmark = pytest.mark.gpu


def _random_case(seed, B, gamma, V, H, r, dtype, w_sd, gumbel, U_sd=2.0):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=H, r=r, dtype=dtype, w_sd=w_sd, U_sd=U_sd, wc_sd=0.05,
                           gumbel=gumbel, seed=seed)
    w = synth.sampler_weights(s)
    w["b_conf"] = 0.25
    x = synth.sampler_batch(s)
    return x, w


def test_tiny_workload_with_logits():
    s = synth.SAMPLER_TINY
    w, x = synth.sampler_weights(s), synth.sampler_batch(s)
    got, ref, ties = sampler_parity(x, w, want_logits=True)
    print(f"tiny: {ties} near-tie steps")


@pytest.mark.parametrize(
    "B,gamma,V,H,r,dtype,w_sd,gumbel",
    [
        (1, 7, 4099, 64, 32, "bf16", 0.5, False),  # ragged V, strong bias
        (3, 1, 1000, 16, 256, "bf16", 0.5, True),  # gamma = 1, Gumbel
        (2, 5, 777, 0, 8, "f32", 0.5, False),  # no hidden part, 32-byte rows
        (17, 3, 2053, 32, 64, "bf16", 0.3, True),  # B spans several request groups
        (5, 4, 513, 8, 3, "f32", 0.5, False),  # rank 3: rows not 16-byte multiples
        (1, 16, 8192, 128, 256, "f32", 0.2, False),  # training block width, fp32 rank 256
        (64, 2, 1024, 16, 256, "bf16", 0.5, True),  # 64 requests
        (2, 3, 1, 4, 16, "bf16", 0.5, False),  # single-token vocabulary
        # single request, bf16, rank 256: the persistent chain kernel
        (1, 7, 1000, 16, 256, "bf16", 0.5, True),  # few workgroups, Gumbel
        (1, 5, 70001, 72, 256, "bf16", 0.3, False),  # ragged slices, H not a multiple of 64
        (1, 5, 3001, 13, 256, "bf16", 0.4, False),  # H not a multiple of 8: the hidden dot's element loop
        (1, 9, 163200, 8, 256, "bf16", 0.2, False),  # largest vocabulary held on chip, gamma above the screen
        (1, 4, 200003, 8, 256, "bf16", 0.2, True),  # beyond it: per-step kernels
        (1, 2, 1, 8, 256, "bf16", 0.5, False),  # single-token vocabulary
        # batched bf16 rank 256: matrix-core step kernel
        (16, 4, 4099, 32, 256, "bf16", 0.5, False),  # one 32-request tile, ragged vocabulary
        (33, 3, 1000, 16, 256, "bf16", 0.5, True),  # two tiles, padded
        (100, 2, 2053, 16, 256, "bf16", 0.3, True),  # two request blocks
        (20, 20, 700, 8, 256, "bf16", 0.5, False),  # gamma above 16: confidences in two rounds
        (3, 18, 500, 8, 32, "f32", 0.5, False),  # same on the vector path
    ],
)
def test_shapes(B, gamma, V, H, r, dtype, w_sd, gumbel):
    x, w = _random_case(0xC0FFEE + B * 131 + V, B, gamma, V, H, r, dtype, w_sd, gumbel)
    sampler_parity(x, w, want_logits=True)



@pytest.mark.parametrize(
    "B,gamma,V,H,gumbel",
    [
        (16, 4, 4096, 32, False),  # one 32-request tile, greedy, whole tiles
        (24, 3, 4104, 13, True),  # ragged last tile, hidden size not a multiple of 8
        (33, 3, 1000, 16, True),  # two request tiles, fewer workgroups than requests
        (64, 5, 12000, 40, False),  # 64 requests, greedy
        (20, 20, 712, 8, False),  # long block
        (48, 2, 65536, 64, True),  # some waves hold fewer tiles than others
        (40, 3, 4100, 13, True),  # V % 8 = 4: the per-step matrix-core kernel instead
    ],
)
def test_batched_without_stored_logits(B, gamma, V, H, gumbel):
    """bf16 rank 256 with 16..64 requests and no stored logits or bias: the
    persistent kernel that keeps W2 in registers and LDS (its U loads take
    16-byte pieces, so it needs V % 8 = 0; other vocabularies take the
    per-step kernel)."""
    x, w = _random_case(0xBA7C4 + B * 131 + V, B, gamma, V, H, 256, "bf16", 0.4, gumbel)
    ws = torch.zeros(dh.head_sample_workspace_size(B, gamma, V, H, 256), dtype=torch.uint8, device="cuda")
    sampler_parity(x, w, want_logits=False, workspace=ws)
    st, paths = dh.workspace_status(ws)
    assert st == 0
    assert bool(paths & dh.PATH_RESIDENT) == (V % 8 == 0), paths
    assert workspace_dirty_bytes(ws) == 0


def test_all_equal_scores_pick_token_zero():
    B, gamma, V, H, r = 3, 4, 3000, 8, 32
    x = {"U": np.zeros((B, gamma, V), np.float32), "h": np.zeros((B, gamma, H), np.float32),
         "x0": np.array([0, 1234, 2999], np.int32)}
    w = {"W1": np.ones((V, r), np.float32), "W2": np.zeros((V, r), np.float32),
         "w_conf": np.zeros(H + r, np.float32), "b_conf": 0.0}
    got, ref, _ = sampler_parity(x, w)
    assert np.all(got["tokens"] == 0)


def test_invalid_token_ids_poison_only_their_request():
    s = synth.SamplerShape(B=4, gamma=3, V=500, H=8, r=16, dtype="f32", w_sd=0.3, U_sd=2.0, wc_sd=0.05,
                           gumbel=False, seed=99)
    w, x = synth.sampler_weights(s), synth.sampler_batch(s)
    x["x0"][1] = -1
    x["x0"][2] = 500
    force = np.full((4, 3), -1, np.int32)
    force[3, 0] = 10_000  # out of range from step 2 on
    out = dh.head_sample(dev(x["U"]), dev(x["h"]), dev(w["W1"]), dev(w["W2"]), dev(w["w_conf"]), 0.0, dev(x["x0"]),
                         force=dev(force))
    tok, conf, surv = (out[k].cpu().numpy() for k in ("tokens", "conf", "survival"))
    assert np.all(tok[1:3] == -1) and np.all(np.isnan(conf[1:3])) and np.all(np.isnan(surv[1:3]))
    assert tok[3, 0] >= 0 and np.all(tok[3, 1:] == -1) and np.isnan(conf[3, 1:]).all() and np.isfinite(conf[3, 0])
    ref = oracle.head_sample(x["U"][:1], x["h"][:1], w["W1"], w["W2"], w["w_conf"], 0.0, x["x0"][:1])
    np.testing.assert_array_equal(tok[0], ref["tokens"][0])


def test_empty_problem_is_a_noop():
    z = torch.zeros((0, 7, 16), device="cuda")
    out = dh.head_sample(z, torch.zeros((0, 7, 4), device="cuda"), torch.zeros((16, 4), device="cuda"),
                         torch.zeros((16, 4), device="cuda"), torch.zeros(8, device="cuda"), 0.0,
                         torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out["tokens"].shape == (0, 7)


def test_repeat_runs_are_bitwise_identical():
    x, w = _random_case(7, 17, 4, 5000, 32, 256, "bf16", 0.3, True)
    a = dh.head_sample(*(dev(v) for v in (x["U"], x["h"], w["W1"], w["W2"], w["w_conf"])), 0.1, dev(x["x0"]),
                       dev(x["G"]), want_logits=True)
    b = dh.head_sample(*(dev(v) for v in (x["U"], x["h"], w["W1"], w["W2"], w["w_conf"])), 0.1, dev(x["x0"]),
                       dev(x["G"]), want_logits=True)
    for k in a:
        assert torch.equal(a[k].view(torch.int32) if a[k].dtype == torch.float32 else a[k],
                           b[k].view(torch.int32) if b[k].dtype == torch.float32 else b[k]), k


def test_single_request_full_vocabulary():
    """B=1, V=151936, H=5120, r=256, bf16, greedy: three seeded anchors."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s)
    total_ties = 0
    for anchor in range(3):
        x = synth.sampler_batch(s, batch_id=anchor)
        _, _, ties = sampler_parity(x, w, want_logits=(anchor == 0))
        total_ties += ties
    print(f"B=1 full vocabulary: {total_ties} near-tie steps over 3 anchors")


def test_single_request_strong_bias():
    """Full vocabulary with a bias large enough to decide most tokens."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s, w_sd=0.5)
    x = synth.sampler_batch(s, batch_id=11)
    got, ref, _ = sampler_parity(x, w)
    plain = np.argmax(synth.bf16_to_f32(x["U"][0]), axis=1)
    assert np.mean(plain != ref["tokens"][0]) > 0.5  # the Markov chain does decide here


@pytest.mark.parametrize("factor", [2.0, 4.0])
def test_single_request_outsized_rows_rebuild_the_screen_table(factor):
    """Trained output factors have heavy-tailed row norms.  A few W2 rows
    with `factor` times the typical norm, at rows the screen's norm sample
    (every V/64-th row) does not read: the screen's guess of the largest row
    norm is too small, so its step table is rebuilt with the measured norm
    (path flag 1; at 4x the windows no longer cover the bound and the block
    moves on to the grid-wide exchange, flag 2).  Tokens, confidences and
    survival still match the oracle."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s)
    rows = np.array([777, 50001, 100003, s.V - 1])
    assert np.all(rows % (s.V // 64) != 0)
    W2 = synth.bf16_to_f32(w["W2"])
    W2[rows] *= factor
    w["W2"] = synth.f32_to_bf16(W2)
    ws = torch.zeros(dh.head_sample_workspace_size(1, s.gamma, s.V, s.H, s.r), dtype=torch.uint8, device="cuda")
    seen = 0
    for anchor in (0, 4):
        sampler_parity(synth.sampler_batch(s, batch_id=anchor), w, workspace=ws)
        st, paths = dh.workspace_status(ws)
        assert st == 0
        assert paths & dh.PATH_B1_REBUILD, paths
        seen |= paths
    print(f"factor {factor}: path flags {seen}")
    assert workspace_dirty_bytes(ws) == 0


def test_single_request_gumbel_screened():
    """B=1 full vocabulary with Gumbel noise and the weak bias of the
    workload: every step is settled by the candidate screen."""
    b1 = synth.SAMPLER_B1
    s = synth.SamplerShape(B=1, gamma=b1.gamma, V=b1.V, H=b1.H, r=b1.r, dtype=b1.dtype, w_sd=b1.w_sd, U_sd=b1.U_sd,
                           wc_sd=b1.wc_sd, gumbel=True, seed=b1.seed + 77)
    w = synth.sampler_weights(s)
    for anchor in range(2):
        sampler_parity(synth.sampler_batch(s, batch_id=anchor), w)


def test_single_request_flat_step_falls_back_mid_block():
    """A step whose base logits are flat over the whole vocabulary has far
    more candidates than the per-workgroup lists hold; the block is finished
    by the grid-wide exchange from that step on."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s)
    x = synth.sampler_batch(s, batch_id=5)
    x["U"][0, 3, :] = synth.f32_to_bf16(np.full(s.V, 5.0, np.float32))
    got, ref, ties = sampler_parity(x, w)
    print(f"flat step 3: {ties} near-tie steps")


def test_single_request_teacher_forced_screened():
    """Forced tokens on the screened path: valid ones replace the sampled
    token as the next step's previous token; an out-of-range one ends the
    block's chain (tokens -1, confidences NaN)."""
    s = synth.SAMPLER_B1
    w = synth.sampler_weights(s)
    x = synth.sampler_batch(s, batch_id=9)
    force = np.full((1, s.gamma), -1, np.int32)
    force[0, 1] = 1234
    force[0, 3] = s.V - 1
    got = run_gpu_sampler(x, w, force, want_logits=False)
    ref = oracle.head_sample(x["U"], x["h"], w["W1"], w["W2"], w["w_conf"], w["b_conf"], x["x0"], None, force)
    for k in range(s.gamma):
        if got["tokens"][0, k] != ref["tokens"][0, k]:
            assert ref["margin"][0, k] < 1e-3, k
            break
        assert abs(got["conf"][0, k] - ref["conf"][0, k]) <= 1e-4
        assert abs(got["survival"][0, k] - ref["survival"][0, k]) <= 1e-4
    force[0, 2] = s.V + 5
    got = run_gpu_sampler(x, w, force, want_logits=False)
    assert np.all(got["tokens"][0, 3:] == -1) and np.isnan(got["conf"][0, 3:]).all()
    assert np.all(got["tokens"][0, :3] >= 0) and np.isfinite(got["conf"][0, :3]).all()


def test_batched_gumbel_full_vocabulary_every_request():
    """B=64 Gumbel-max at full size, all 64 requests in one call (the resident
    kernel the benchmark times); the oracle checks every request under the
    near-tie protocol (about 9 s of oracle time)."""
    s = synth.SAMPLER_B64
    w = synth.sampler_weights(s)
    x = synth.sampler_batch(s)
    got, ref, ties = sampler_parity(x, w)
    assert ties <= 2
    assert np.all(got["tokens"] >= 0)


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves calls of different batch sizes,
    vocabulary sizes and block widths, on every kernel path (single-request
    screen and exchange, matrix cores resident and per step, vector); each
    call leaves it zeroed."""
    cases = [(1, 151936, 7, False, 0.02), (64, 151936, 7, True, 0.02), (1, 1000, 3, True, 0.3),
             (17, 4096, 5, False, 0.3), (1, 70001, 9, False, 0.3), (64, 151936, 3, False, 0.02),
             (1, 151936, 7, True, 0.02), (5, 3000, 4, True, 0.3)]
    big = max(dh.head_sample_workspace_size(B, g, V, 64, 256) for B, V, g, _, _ in cases)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for i, (B, V, gamma, gumbel, w_sd) in enumerate(cases):
        s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=64, r=256, dtype="bf16", w_sd=w_sd, U_sd=2.0, wc_sd=0.05,
                               gumbel=gumbel, seed=500 + i)
        w, x = synth.sampler_weights(s), synth.sampler_batch(s)
        args = [dev(v) for v in (x["U"], x["h"], w["W1"], w["W2"], w["w_conf"])] + [0.1, dev(x["x0"]), dev(x["G"])]
        a = dh.head_sample(*args, workspace=ws)
        b = dh.head_sample(*args)
        for k in a:
            assert torch.equal(a[k], b[k]), (B, V, k)
        assert workspace_dirty_bytes(ws) == 0, (B, V, gamma)


@pytest.mark.parametrize("gumbel", [False, True])
def test_gated_head_tiny(gumbel):
    """Gated Markov head on the tiny fp32 workload (general path), with the
    stored logits and bias compared too."""
    s = synth.SAMPLER_TINY
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 0.1))
    x = synth.sampler_batch(s)
    if gumbel:
        x["G"] = synth.gumbel(synth.key(s.seed, 99), x["U"].shape)
    else:
        x.pop("G", None)
    sampler_parity(x, w, want_logits=True)


@pytest.mark.parametrize("B,V,gamma,H,r", [(5, 30001, 5, 512, 64), (1, 4099, 9, 96, 32), (17, 2000, 3, 64, 8),
                                           (3, 2000, 4, 60, 12)])  # the last: generic gate step (r % 8 != 0)
def test_gated_head_bf16_shapes(B, V, gamma, H, r):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=H, r=r, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=True, seed=synth.SEED_BASE + 40 + V)
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 1.0 / np.sqrt(H + r)))
    x = synth.sampler_batch(s)
    sampler_parity(x, w, want_logits=True)


def test_gated_head_full_vocabulary():
    """The serving shape's weights (V=151936, H=5120, r=256, bf16), 8 requests,
    Gumbel-max; every request checked."""
    s = synth.SAMPLER_B64
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 0.02))
    x = synth.sampler_batch(s, B=8)
    _, _, ties = sampler_parity(x, w)
    assert ties <= 1


@pytest.mark.parametrize("B,V,gamma", [(16, 4099, 3), (40, 30001, 5)])
def test_gated_head_matrix_core_shapes(B, V, gamma):
    """Rank 256 and B >= 16 in bf16 put the gated head's bias on the matrix
    cores (one and two 32-request tiles, ragged vocabulary tail); stored logits
    and bias compared too."""
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=256, r=256, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=True, seed=synth.SEED_BASE + 140 + V)
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 1.0 / np.sqrt(512)))
    x = synth.sampler_batch(s)
    sampler_parity(x, w, want_logits=True)


def test_gated_head_batched_serving_workload():
    """B=64 at the serving shape (V=151936, H=5120, r=256, bf16, Gumbel-max) in
    the launch configuration the benchmark times; every request checked and
    the workspace left zero."""
    s = synth.SAMPLER_B64
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 0.02))
    x = synth.sampler_batch(s)
    n = dh.lib().dspark_head_sample_gated_workspace_size(64, 7, s.V, s.H, s.r, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    _, _, ties = sampler_parity(x, w, workspace=ws)
    assert ties <= 2
    assert workspace_dirty_bytes(ws) == 0


def test_gated_head_leaves_workspace_zero():
    s = synth.SamplerShape(B=3, gamma=4, V=5000, H=64, r=16, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=False, seed=synth.SEED_BASE + 77)
    w = dict(synth.sampler_weights(s), Wg=synth.gate_weights(s, 0.1))
    x = synth.sampler_batch(s)
    n = dh.lib().dspark_head_sample_gated_workspace_size(3, 4, 5000, 64, 16, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    args = [dev(x["U"]), dev(x["h"]), dev(w["W1"]), dev(w["W2"]), dev(w["w_conf"]), w["b_conf"], dev(x["x0"])]
    a = dh.head_sample(*args, Wg=dev(w["Wg"]), workspace=ws)
    assert workspace_dirty_bytes(ws) == 0
    b = dh.head_sample(*args, Wg=dev(w["Wg"]))
    assert torch.equal(a["tokens"], b["tokens"]) and torch.equal(a["conf"], b["conf"])


@pytest.mark.parametrize("head", ["gated", "rnn"])
@pytest.mark.parametrize("gumbel", [False, True])
def test_gated_and_rnn_heads_on_the_resident_kernel(head, gumbel):
    """B=40 (two 32-request blocks) at V=30000, rank 256, bf16: the gated and
    RNN heads run in the resident-W2 kernel, where each workgroup forms one
    column of the head's embedding per step and reads the others back; every
    request checked, the path flag and a zero workspace verified."""
    s = synth.SamplerShape(B=40, gamma=5, V=30000, H=256, r=256, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=gumbel, seed=synth.SEED_BASE + 180 + int(gumbel) + (2 if head == "rnn" else 0))
    w = synth.sampler_weights(s)
    if head == "gated":
        w["Wg"] = synth.gate_weights(s, 1.0 / np.sqrt(512))
        n = dh.lib().dspark_head_sample_gated_workspace_size(40, 5, 30000, 256, 256, 1)
    else:
        w["Wr"] = synth.rnn_weights(s, 1.0 / np.sqrt(768))
        n = dh.lib().dspark_head_sample_rnn_workspace_size(40, 5, 30000, 256, 256, 1)
    x = synth.sampler_batch(s)
    if not gumbel:
        x.pop("G", None)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    sampler_parity(x, w, workspace=ws)
    st, paths = dh.workspace_status(ws)
    assert st == 0
    if torch.cuda.get_device_properties(0).multi_processor_count >= 256:  # a workgroup per rank column
        assert paths & dh.PATH_RESIDENT
    assert workspace_dirty_bytes(ws) == 0


@pytest.mark.parametrize("gumbel", [False, True])
def test_rnn_head_tiny(gumbel):
    """RNN head on the tiny fp32 workload (general path), stored logits and
    bias compared too."""
    s = synth.SAMPLER_TINY
    w = dict(synth.sampler_weights(s), Wr=synth.rnn_weights(s, 0.08))
    x = synth.sampler_batch(s)
    if gumbel:
        x["G"] = synth.gumbel(synth.key(s.seed, 97), x["U"].shape)
    sampler_parity(x, w, want_logits=True)


@pytest.mark.parametrize("B,V,gamma,H,r", [(5, 30001, 5, 512, 64), (1, 4099, 9, 96, 32), (17, 2000, 3, 64, 8),
                                           (3, 2000, 4, 60, 12)])  # the last: generic state step (r % 8 != 0)
def test_rnn_head_bf16_shapes(B, V, gamma, H, r):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=H, r=r, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=True, seed=synth.SEED_BASE + 60 + V)
    w = dict(synth.sampler_weights(s), Wr=synth.rnn_weights(s, 1.0 / np.sqrt(2 * r + H)))
    x = synth.sampler_batch(s)
    sampler_parity(x, w, want_logits=True)


@pytest.mark.parametrize("B,V,gamma", [(16, 4099, 3), (40, 30001, 5)])
def test_rnn_head_matrix_core_shapes(B, V, gamma):
    s = synth.SamplerShape(B=B, gamma=gamma, V=V, H=256, r=256, dtype="bf16", w_sd=0.3, U_sd=1.0, wc_sd=0.02,
                           gumbel=True, seed=synth.SEED_BASE + 160 + V)
    w = dict(synth.sampler_weights(s), Wr=synth.rnn_weights(s, 1.0 / np.sqrt(768)))
    x = synth.sampler_batch(s)
    sampler_parity(x, w, want_logits=True)


def test_rnn_head_batched_serving_workload():
    """B=64 at the serving shape in the benchmark's launch configuration;
    every request checked and the workspace left zero."""
    s = synth.SAMPLER_B64
    w = dict(synth.sampler_weights(s), Wr=synth.rnn_weights(s, 0.015))
    x = synth.sampler_batch(s)
    n = dh.lib().dspark_head_sample_rnn_workspace_size(64, 7, s.V, s.H, s.r, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    _, _, ties = sampler_parity(x, w, workspace=ws)
    assert ties <= 2
    assert workspace_dirty_bytes(ws) == 0


def test_rnn_head_full_vocabulary_and_workspace():
    """The serving shape's weights (V=151936, H=5120, r=256, bf16), 8 requests,
    Gumbel-max, every request checked; the workspace is left zero."""
    s = synth.SAMPLER_B64
    w = dict(synth.sampler_weights(s), Wr=synth.rnn_weights(s, 0.015))
    x = synth.sampler_batch(s, B=8)
    _, _, ties = sampler_parity(x, w)
    assert ties <= 1
    n = dh.lib().dspark_head_sample_rnn_workspace_size(8, 7, s.V, s.H, s.r, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dh.head_sample(dev(x["U"]), dev(x["h"]), dev(w["W1"]), dev(w["W2"]), dev(w["w_conf"]), w["b_conf"],
                   dev(x["x0"]), dev(x["G"]), Wr=tuple(dev(a) for a in w["Wr"]), workspace=ws)
    assert workspace_dirty_bytes(ws) == 0
