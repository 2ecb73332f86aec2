"""Benchmark of the draft-head hot path on one MI355X.

One step is one serving round of the full-vocabulary single-request workload
(B=1, gamma=7, V=151936, H=5120, r=256, bf16 weights, greedy argmax): the
Markov-head block sampler with its confidence head and survival products is
called once for each of 1000 seeded anchors, back to back, then the prefix
scheduler runs once over the 1000 x 7 confidences.  `value` is draft
positions per second (bias + sample + confidence) over the timed steps.

The same run also times the analytic accept rate on the training-width
workload (2048 positions x V=151936, bf16) and reports it as GB/s under
`accept_rate`, and times the CPU oracle on a bounded sample of the step
(`cpu_baseline`).  Inputs are synthetic (seeded generator), resident in HBM
before the timed region starts.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--anchors 1000]
                       [--no-cpu] [--no-accept] [--extra]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0


def to_dev(a, device):
    import numpy as np
    import torch

    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def sampler_call_bytes(B, gamma, V, H, r, elem=2):
    """Compulsory HBM bytes of one sampler call: W2 once, U, gathered W1
    rows, h, w_conf, anchors, and the three [B, gamma] outputs."""
    return (V * r + B * gamma * V + B * gamma * r + B * gamma * H + (H + r)) * elem + 4 * B + 12 * B * gamma


def accept_call_bytes(N, V, elem=2):
    return 2 * N * V * elem + 4 * N


def verify_call_bytes(n_draft, all_kept, V, gamma, elem=2):
    """Unique bytes of one verify call: the draft and target rows of every
    drafted position once, the target row of the bonus position for requests
    that kept every drafted token, each request's Gumbel row, and the small
    per-position inputs and outputs.  (The rows of a rejected position are
    read a second time for the residual draw; that is in `traffic`.)"""
    import numpy as np

    n = np.asarray(n_draft, np.int64)
    B = n.size
    rows = int(n.sum()) * 2 + int(np.asarray(all_kept).sum())
    return rows * V * elem + B * V * 4 + B * gamma * 8 + B * 12


def profiled_traffic(profile: str, sources: list[str]):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counter
    passes recorded in profiles/<profile>, or None when the kernel sources
    changed since those counters were taken (hash mismatch) or no record
    exists."""
    import hashlib

    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if rec.get("source_sha256") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in rec:
        return None
    return int(float(rec["traffic_bytes_per_launch"]))


SAMPLER_SOURCES = ["draft_head_sampling_amd/csrc/head_sample.hip", "draft_head_sampling_amd/csrc/internal.h"]
VERIFY_SOURCES = ["draft_head_sampling_amd/csrc/verify.hip", "draft_head_sampling_amd/csrc/internal.h"]
ACCEPT_SOURCES = ["draft_head_sampling_amd/csrc/accept_rate.hip", "draft_head_sampling_amd/csrc/internal.h"]
LOSS_SOURCES = ["draft_head_sampling_amd/csrc/block_loss.hip", "draft_head_sampling_amd/csrc/block_loss.h",
                "draft_head_sampling_amd/csrc/internal.h"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--anchors", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-accept", action="store_true", help="skip the accept-rate measurement")
    ap.add_argument("--no-verify", action="store_true", help="skip the rejection-sampling verify measurement")
    ap.add_argument("--extra", action="store_true", help="also time the B=64 sampler and the scheduler workload")
    ap.add_argument("--calib-copy", action="store_true", help="run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache sampler timing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the draft-head path is data-parallel by request and this build runs "
              "on a single MI355X; --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_head_sampling_amd as dh
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dh.lib()  # fails loudly if the HIP library is missing
    stream = torch.cuda.current_stream(dev)

    # ---------------- inputs (host generation, then resident in HBM) ----------------
    s = synth.SAMPLER_B1
    n_anch = args.anchors
    w = synth.sampler_weights(s)
    W = {k: to_dev(v, dev) for k, v in w.items() if k != "b_conf"}
    U = torch.empty((n_anch, s.gamma, s.V), dtype=torch.bfloat16, device=dev)
    Hh = torch.empty((n_anch, s.gamma, s.H), dtype=torch.bfloat16, device=dev)
    X0 = torch.empty((n_anch,), dtype=torch.int32, device=dev)
    host_batches = []
    for a in range(n_anch):
        x = synth.sampler_batch(s, batch_id=a)
        U[a].copy_(to_dev(x["U"][0], dev))
        Hh[a].copy_(to_dev(x["h"][0], dev))
        X0[a : a + 1].copy_(torch.from_numpy(x["x0"]))
        if a < 64:
            host_batches.append(x)
    tokens = torch.empty((n_anch, s.gamma), dtype=torch.int32, device=dev)
    conf = torch.empty((n_anch, s.gamma), dtype=torch.float32, device=dev)
    surv = torch.empty((n_anch, s.gamma), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(dh.head_sample_workspace_size(1, s.gamma, s.V, s.H, s.r), 256), dtype=torch.uint8,
                     device=dev)
    calls = []
    for a in range(n_anch):
        c, _ = dh.prepare_head_sample(U[a : a + 1], Hh[a : a + 1], W["W1"], W["W2"], W["w_conf"], w["b_conf"],
                                      X0[a : a + 1], tokens=tokens[a : a + 1], conf=conf[a : a + 1],
                                      survival=surv[a : a + 1], workspace=ws)
        calls.append(c)
    n_sps = n_anch * (s.gamma + 1)
    sps_host = synth.sps_table(n_sps, "steps")
    sps = to_dev(sps_host, dev)
    sched, sched_out = dh.prepare_prefix_schedule(conf, sps, want_order=False)
    torch.cuda.synchronize()

    e_s0 = torch.cuda.Event(enable_timing=True)
    e_s1 = torch.cuda.Event(enable_timing=True)
    samp_ms = []

    def step(record):
        if record:
            e_s0.record(stream)
        for c in calls:
            c()
        if record:
            e_s1.record(stream)
        sched()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()  # harvest the sampler-only interval of this step
        samp_ms.append(e_s0.elapsed_time(e_s1))
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    positions = n_anch * s.gamma
    value = positions * args.steps / (total_ms / 1e3)

    call_us = float(np.mean(samp_ms)) * 1e3 / n_anch
    call_bytes = sampler_call_bytes(1, s.gamma, s.V, s.H, s.r)
    achieved = call_bytes / (call_us * 1e-6) / 1e9

    line = {
        "metric": "draft positions/sec (bias+sample+conf) and accept-rate GB/s vs HBM roofline",
        "value": round(value, 1),
        "unit": "draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded SplitMix64/Box-Muller), random weights",
        "config": {
            "workload": f"Markov-head block sampler, {n_anch} anchors back to back, B=1 gamma=7 V=151936 H=5120 "
                        f"r=256 bf16 greedy + prefix scheduler over {n_anch}x7 confidences",
            "B": 1, "gamma": s.gamma, "V": s.V, "H": s.H, "r": s.r, "anchors_per_step": n_anch,
        },
        "roofline": {
            "kernel": "dspark_head_sample (one call = one anchor)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic("head_sample_chain_b1_vocab151936.md", SAMPLER_SOURCES),
            "bytes_per_launch": call_bytes,
            "us_per_launch": round(call_us, 3),
        },
        "wall_s": round(wall, 3),
    }

    # ---------------- cold caches: a 512 MiB write before each call ----------------
    # W2 (77.8 MB) fits the 256 MB Infinity Cache, so back-to-back calls read
    # it from there; here every call first finds the caches full of other
    # data, and HIP events bracket the call alone.
    scrub = None
    if not args.no_cold:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for i, (c0, c1) in enumerate(ev):
            scrub.fill_(i & 0xFF)
            c0.record(stream)
            calls[i % n_anch]()
            c1.record(stream)
        torch.cuda.synchronize()
        cold = sorted(c0.elapsed_time(c1) * 1e3 for c0, c1 in ev)
        line["cold"] = {"b1_us_per_call_median": round(cold[len(cold) // 2], 2), "calls": len(cold),
                        "scrub_bytes": 512 << 20}

    # ---------------- accept rate on the training-width workload ----------------
    if not args.no_accept:
        sa = synth.ACCEPT_TRAIN
        d, t = synth.accept_inputs(sa)
        D, T = to_dev(d, dev), to_dev(t, dev)
        del d, t
        acall, aout = dh.prepare_accept_rate(D, T)
        for _ in range(3):
            acall()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        reps = 20
        a0.record(stream)
        for _ in range(reps):
            acall()
        a1.record(stream)
        torch.cuda.synchronize()
        a_us = a0.elapsed_time(a1) * 1e3 / reps
        a_bytes = accept_call_bytes(sa.N, sa.V)
        gbs = a_bytes / (a_us * 1e-6) / 1e9
        line["accept_rate"] = {
            "value": round(gbs, 1), "unit": "GB/s",
            "workload": "analytic accept rate, 2048 positions x V=151936 bf16 draft/target logits",
            "us_per_call": round(a_us, 2), "positions_per_s": round(sa.N / (a_us * 1e-6), 1),
            "roofline": {"kernel": "dspark_accept_rate", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("accept_rate_cluster_2048x151936.md", ACCEPT_SOURCES),
                         "bytes_per_launch": a_bytes},
        }
        del D, T

    # ---------------- rejection-sampling verify on the batched serving shape ----------------
    if not args.no_verify:
        sv = synth.VERIFY_B64
        vin = synth.verify_inputs(sv)
        vd = {k: to_dev(v, dev) for k, v in vin.items()}
        del vin
        vcall, vout = dh.prepare_verify(vd["d"], vd["t"], vd["x"], vd["u"], vd["G"])
        for _ in range(3):
            vcall()
        torch.cuda.synchronize()
        v0 = torch.cuda.Event(enable_timing=True)
        v1 = torch.cuda.Event(enable_timing=True)
        reps = 20
        v0.record(stream)
        for _ in range(reps):
            vcall()
        v1.record(stream)
        torch.cuda.synchronize()
        v_us = v0.elapsed_time(v1) * 1e3 / reps
        n_acc = vout["n_accepted"].cpu().numpy()
        v_bytes = verify_call_bytes([sv.gamma] * sv.B, n_acc == sv.gamma, sv.V, sv.gamma)
        v_gbs = v_bytes / (v_us * 1e-6) / 1e9
        line["verify"] = {
            "workload": "rejection-sampling verify, B=64 requests x 7 drafted positions, V=151936 bf16 draft and "
                        "target logits, fp32 uniforms and Gumbel rows",
            "us_per_call": round(v_us, 2), "positions_per_s": round(sv.B * sv.gamma / (v_us * 1e-6), 1),
            "mean_accepted": round(float(n_acc.mean()), 3),
            "roofline": {"kernel": "dspark_verify (2 launches; verify_stats reads every drafted row)",
                         "bound": "hbm", "achieved": round(v_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(v_gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("verify_b64_vocab151936.md", VERIFY_SOURCES),
                         "bytes_per_launch": v_bytes},
        }
        del vd

    if args.extra:
        s3 = synth.SAMPLER_B64
        x3 = synth.sampler_batch(s3)
        c3, _ = dh.prepare_head_sample(to_dev(x3["U"], dev), to_dev(x3["h"], dev), W["W1"], W["W2"], W["w_conf"],
                                       0.0, to_dev(x3["x0"], dev), to_dev(x3["G"], dev))
        for _ in range(3):
            c3()
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(10):
            c3()
        b1.record(stream)
        torch.cuda.synchronize()
        us3 = b0.elapsed_time(b1) * 1e3 / 10
        if scrub is not None:  # the same call with cold caches
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
            for i, (c0, c1) in enumerate(ev):
                scrub.fill_(i & 0xFF)
                c0.record(stream)
                c3()
                c1.record(stream)
            torch.cuda.synchronize()
            cold3 = sorted(c0.elapsed_time(c1) * 1e3 for c0, c1 in ev)
            line["cold"]["b64_us_per_call_median"] = round(cold3[len(cold3) // 2], 2)
        flops = 2.0 * 64 * s3.gamma * s3.V * s3.r
        by3 = sampler_call_bytes(64, 7, s3.V, s3.H, s3.r) + 64 * 7 * s3.V * 4
        gb3 = by3 / (us3 * 1e-6) / 1e9
        line["extra_b64"] = {"workload": "Markov-head block sampler, B=64 gamma=7 V=151936 H=5120 r=256 bf16, "
                                         "Gumbel-max with fp32 noise",
                             "us_per_call": round(us3, 2), "positions_per_s": round(64 * 7 / (us3 * 1e-6), 1),
                             "mfma_tflops": round(flops / (us3 * 1e-6) / 1e12, 2),
                             "roofline": {"kernel": "dspark_head_sample B=64 (one resident kernel)",
                                          "bound": "hbm", "achieved": round(gb3, 1), "peak": HBM_PEAK_GBS,
                                          "unit": "GB/s", "frac": round(gb3 / HBM_PEAK_GBS, 4),
                                          "traffic": profiled_traffic("head_sample_resident_b64_vocab151936.md",
                                                                      SAMPLER_SOURCES),
                                          "bytes_per_launch": by3}}
        # the gated Markov head on the same batch (per-step path on the matrix cores)
        Wg3 = to_dev(synth.gate_weights(s3, 0.02), dev)
        cg, _ = dh.prepare_head_sample(to_dev(x3["U"], dev), to_dev(x3["h"], dev), W["W1"], W["W2"], W["w_conf"],
                                       0.0, to_dev(x3["x0"], dev), to_dev(x3["G"], dev), Wg=Wg3)
        for _ in range(2):
            cg()
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(5):
            cg()
        b1.record(stream)
        torch.cuda.synchronize()
        usg = b0.elapsed_time(b1) * 1e3 / 5
        byg = by3 + s3.r * (s3.H + s3.r) * 2
        gbg = byg / (usg * 1e-6) / 1e9
        line["extra_gated_b64"] = {
            "workload": "gated Markov head, B=64 gamma=7 V=151936 H=5120 r=256 bf16, Gumbel-max with fp32 noise",
            "us_per_call": round(usg, 2), "positions_per_s": round(64 * 7 / (usg * 1e-6), 1),
            "roofline": {"kernel": "dspark_head_sample_gated (per-step matrix-core path: gate and bias "
                                   "kernels per position)",
                         "bound": "hbm", "achieved": round(gbg, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbg / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("head_sample_gated_b64_vocab151936.md", SAMPLER_SOURCES),
                         "bytes_per_launch": byg}}
        # the RNN head on the same batch (per-step path on the matrix cores)
        Wr3 = tuple(to_dev(a, dev) for a in synth.rnn_weights(s3, 0.015))
        cr, _ = dh.prepare_head_sample(to_dev(x3["U"], dev), to_dev(x3["h"], dev), W["W1"], W["W2"], W["w_conf"],
                                       0.0, to_dev(x3["x0"], dev), to_dev(x3["G"], dev), Wr=Wr3)
        for _ in range(2):
            cr()
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(5):
            cr()
        b1.record(stream)
        torch.cuda.synchronize()
        usr = b0.elapsed_time(b1) * 1e3 / 5
        byr = by3 + 2 * s3.r * (2 * s3.r + s3.H) * 2
        gbr = byr / (usr * 1e-6) / 1e9
        line["extra_rnn_b64"] = {
            "workload": "RNN head, B=64 gamma=7 V=151936 H=5120 r=256 bf16, Gumbel-max with fp32 noise",
            "us_per_call": round(usr, 2), "positions_per_s": round(64 * 7 / (usr * 1e-6), 1),
            "roofline": {"kernel": "dspark_head_sample_rnn (per-step matrix-core path: state and bias "
                                   "kernels per position)",
                         "bound": "hbm", "achieved": round(gbr, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbr / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("head_sample_rnn_b64_vocab151936.md", SAMPLER_SOURCES),
                         "bytes_per_launch": byr}}
        s5 = synth.SCHEDULE_TRAIN
        for kind in ("tokens", "steps"):
            c5, _ = dh.prepare_prefix_schedule(to_dev(synth.schedule_conf(s5), dev),
                                               to_dev(synth.sps_table(s5.n_sps, kind), dev))
            for _ in range(5):
                c5()
            torch.cuda.synchronize()
            b0.record(stream)
            for _ in range(50):
                c5()
            b1.record(stream)
            torch.cuda.synchronize()
            line[f"extra_sched_{kind}_us"] = round(b0.elapsed_time(b1) * 1e3 / 50, 2)
        # the teacher-forced block bias with the joint loss at 2048 training positions
        s6 = synth.LOSS_TRAIN
        x6 = synth.loss_inputs(s6)
        d6 = {k: (to_dev(v, dev) if isinstance(v, np.ndarray) else v) for k, v in x6.items()}
        del x6
        c6, _ = dh.prepare_block_loss(d6["U"], d6["t"], d6["h"], d6["W1"], d6["W2"], d6["w_conf"], d6["b_conf"],
                                      d6["xp"], d6["y"])
        for _ in range(2):
            c6()
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(5):
            c6()
        b1.record(stream)
        torch.cuda.synchronize()
        us6 = b0.elapsed_time(b1) * 1e3 / 5
        M6 = s6.N * s6.gamma
        by6 = (2 * M6 * s6.V * 2 + s6.V * s6.r * 2 + M6 * s6.r * 2 + M6 * s6.H * 2 + (s6.H + s6.r) * 2 + 8 * M6
               + 16 * M6 + 16)
        gb6 = by6 / (us6 * 1e-6) / 1e9
        line["extra_block_loss"] = {
            "workload": "teacher-forced block bias + joint loss (CE, L1, confidence BCE), 2048 positions "
                        "(128 anchors x block 16), V=151936 H=5120 r=256 bf16",
            "us_per_call": round(us6, 2), "positions_per_s": round(M6 / (us6 * 1e-6), 1),
            "mfma_tflops": round(2 * M6 * s6.V * s6.r / (us6 * 1e-6) / 1e12, 2),
            "roofline": {"kernel": "dspark_block_loss (two tile passes over U and t, W2 on the matrix cores)",
                         "bound": "hbm", "achieved": round(gb6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gb6 / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("block_loss_2048x151936.md", LOSS_SOURCES),
                         "bytes_per_launch": by6}}
        del d6

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = 1 << 30

    # ---------------- CPU oracle on a bounded sample ----------------
    if not args.no_cpu:
        import oracle

        n_cpu = 0
        tc0 = time.perf_counter()
        while n_cpu < len(host_batches) and (time.perf_counter() - tc0) < 12.0:
            x = host_batches[n_cpu]
            oracle.head_sample(x["U"], x["h"], w["W1"], w["W2"], w["w_conf"], w["b_conf"], x["x0"])
            n_cpu += 1
        t_samp = time.perf_counter() - tc0
        conf_host = conf.cpu().numpy()
        tc1 = time.perf_counter()
        oracle.prefix_schedule(conf_host, sps_host)
        t_sched = time.perf_counter() - tc1
        # one step = n_anch sampler calls + one schedule: scale the sample
        cpu_step_s = t_samp / n_cpu * n_anch + t_sched
        line["cpu_baseline"] = {
            "value": round(positions / cpu_step_s, 2), "unit": "draft positions/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle sampler on {n_cpu} of the {n_anch} anchors ({t_samp:.1f} s, fp64, single thread), "
                      f"scaled to {n_anch}, plus one oracle schedule of the {n_anch}x7 confidences "
                      f"({t_sched * 1e3:.1f} ms); host: {os.cpu_count()} logical CPUs",
        }

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
