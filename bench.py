"""Benchmark of the draft-head hot path on one MI355X.

One step is one serving round of the full-vocabulary single-request workload
(B=1, gamma=7, V=151936, H=5120, r=256, bf16 weights, greedy argmax): the
Markov-head block sampler with its confidence head and survival products is
called once for each of 1000 seeded anchors, back to back, then the prefix
scheduler runs once over the 1000 x 7 confidences.  `value` is draft
positions per second (bias + sample + confidence) over the timed steps.

The same run times every other workload once, each as its own object with an
HBM (or matrix-core) roofline: the B=1 sampler with cold caches and with a
strong Markov bias (the grid-wide exchange path) and with the W2 row-norm
bound computed once per weight load (dspark_w2_bound; its own cost is
reported beside it, and `value` does not use it); the batched Gumbel-max
sampler (B=64) with its matrix-core figures; the gated and RNN heads; the
analytic accept rate on 2048 training positions; the prefix scheduler on 256 x
16 confidences with both throughput tables; rejection-sampling verify; and the
teacher-forced block loss.  The CPU oracle is timed on a bounded sample of the
step, single-threaded and on every host core, and its tokens are compared with
the GPU's.  Inputs are synthetic (seeded generator) and resident in HBM before
any timed region starts.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--anchors 1000]
                       [--legs all|b1,cold,strong,w2bound,accept,verify,b64,gated,rnn,schedule,loss,cpu]
                       [--no-cpu] [--no-accept] [--no-verify] [--no-cold] [--calib-copy]
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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
ALL_LEGS = ("b1", "cold", "strong", "w2bound", "accept", "verify", "b64", "gated", "rnn", "schedule", "loss", "cpu")


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
SCHED_SOURCES = ["draft_head_sampling_amd/csrc/prefix_schedule.hip", "draft_head_sampling_amd/csrc/internal.h"]


def hbm_roofline(kernel, nbytes, us, profile=None, sources=None, cold_us=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    r = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4),
         "traffic": profiled_traffic(profile, sources) if profile else None,
         "bytes_per_launch": int(nbytes), "us_per_launch": round(us, 3)}
    if cold_us is not None:
        cg = nbytes / (cold_us * 1e-6) / 1e9
        r["cold"] = {"us_per_launch": round(cold_us, 3), "achieved": round(cg, 1), "frac": round(cg / HBM_PEAK_GBS, 4)}
    return r


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--anchors", type=int, default=1000)
    ap.add_argument("--legs", default="all", help="comma list of " + ",".join(ALL_LEGS) + " (b1 always runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-accept", action="store_true", help="skip the accept-rate measurement")
    ap.add_argument("--no-verify", action="store_true", help="skip the rejection-sampling verify measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timings")
    ap.add_argument("--calib-copy", action="store_true", help="run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the draft-head path is data-parallel by request and this build runs "
              "on a single MI355X; --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    legs = set(ALL_LEGS) if args.legs == "all" else set(args.legs.split(",")) | {"b1"}
    unknown = legs - set(ALL_LEGS)
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")
    for flag, leg in ((args.no_cpu, "cpu"), (args.no_accept, "accept"), (args.no_verify, "verify"),
                      (args.no_cold, "cold")):
        if flag:
            legs.discard(leg)

    import numpy as np
    import torch

    import draft_head_sampling_amd as dh
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dh.lib()  # fails loudly if the HIP library is missing
    stream = torch.cuda.current_stream(dev)

    def timed(call, reps):
        """Average microseconds per call of `reps` back-to-back calls (HIP
        events on the launch stream)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if "cold" in legs else None

    def timed_cold(call, reps):
        """Median microseconds of one call after a 512 MiB write has evicted
        the caches (W2 would otherwise be re-read from the 256 MB Infinity
        Cache); the events bracket the call alone."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (c0, c1) in enumerate(ev):
            scrub.fill_(i & 0xFF)
            c0.record(stream)
            call()
            c1.record(stream)
        torch.cuda.synchronize()
        t = sorted(c0.elapsed_time(c1) * 1e3 for c0, c1 in ev)
        return t[len(t) // 2]

    # ---------------- B=1 step inputs (host generation, then resident in HBM) ----------------
    s = synth.SAMPLER_B1
    n_anch = args.anchors
    w = synth.sampler_weights(s)
    W = {k: to_dev(v, dev) for k, v in w.items() if k != "b_conf"}
    U = torch.empty((n_anch, s.gamma, s.V), dtype=torch.bfloat16, device=dev)
    Hh = torch.empty((n_anch, s.gamma, s.H), dtype=torch.bfloat16, device=dev)
    X0 = torch.empty((n_anch,), dtype=torch.int32, device=dev)
    host_batches = []
    n_keep = 64
    for a in range(n_anch):
        x = synth.sampler_batch(s, batch_id=a)
        U[a].copy_(to_dev(x["U"][0], dev))
        Hh[a].copy_(to_dev(x["h"][0], dev))
        X0[a : a + 1].copy_(torch.from_numpy(x["x0"]))
        if a < n_keep:
            host_batches.append(x)
    tokens = torch.empty((n_anch, s.gamma), dtype=torch.int32, device=dev)
    conf = torch.empty((n_anch, s.gamma), dtype=torch.float32, device=dev)
    surv = torch.empty((n_anch, s.gamma), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(dh.head_sample_workspace_size(1, s.gamma, s.V, s.H, s.r), 256), dtype=torch.uint8,
                     device=dev)

    def anchor_calls(Wd, tok, cf, sv):
        calls = []
        for a in range(n_anch):
            c, _ = dh.prepare_head_sample(U[a : a + 1], Hh[a : a + 1], Wd["W1"], Wd["W2"], Wd["w_conf"], 0.0,
                                          X0[a : a + 1], tokens=tok[a : a + 1], conf=cf[a : a + 1],
                                          survival=sv[a : a + 1], workspace=ws)
            calls.append(c)
        return calls

    calls = anchor_calls(W, tokens, conf, surv)
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
    st_b1, paths_b1 = dh.workspace_status(ws)
    cold_b1 = timed_cold(lambda: calls[0](), 50) if scrub is not None else None

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
        "roofline": hbm_roofline("dspark_head_sample (one call = one anchor; W2 read once per call)", call_bytes,
                                 call_us, "head_sample_chain_b1_vocab151936.md", SAMPLER_SOURCES, cold_b1),
        "b1_paths": {"give_up": st_b1, "path_flags": paths_b1},
        "wall_s": round(wall, 3),
    }

    # ---------------- B=1 with a strong Markov bias: the grid-wide exchange ----------------
    if "strong" in legs:
        ws_strong = synth.sampler_weights(s, w_sd=0.5)
        Ws = {k: to_dev(v, dev) for k, v in ws_strong.items() if k != "b_conf"}
        tok_s = torch.empty_like(tokens)
        conf_s = torch.empty_like(conf)
        surv_s = torch.empty_like(surv)
        n_str = min(200, n_anch)
        scalls = anchor_calls(Ws, tok_s, conf_s, surv_s)[:n_str]
        dh.workspace_status(ws)  # clear the path flags
        for c in scalls[:10]:
            c()
        torch.cuda.synchronize()
        us_s = timed(lambda: [c() for c in scalls], 1) / n_str
        st_s, paths_s = dh.workspace_status(ws)
        line["b1_strong_bias"] = {
            "workload": f"B=1 gamma=7 V=151936 H=5120 r=256 bf16 greedy, W1 and W2 ~ N(0, 0.5), {n_str} anchors "
                        "back to back: the bias decides most tokens and the steps go to the grid-wide exchange",
            "us_per_call": round(us_s, 3), "positions_per_s": round(s.gamma / (us_s * 1e-6), 1),
            "give_up": st_s, "path_flags": paths_s,
            "roofline": hbm_roofline("dspark_head_sample (persistent kernel, per-step exchange)", call_bytes, us_s,
                                     "head_sample_chain_b1_strong_bias_vocab151936.md", SAMPLER_SOURCES,
                                     timed_cold(lambda: scalls[0](), 20) if scrub is not None else None),
        }
        del Ws

    # ---------------- B=1 with the weights-only W2 bound computed once per weight load ----------------
    if "w2bound" in legs:
        bound = dh.w2_bound(W["W2"])
        L_ = dh.lib()
        w2p, bp = W["W2"].data_ptr(), bound.data_ptr()
        bound_us = timed(lambda: L_.dspark_w2_bound(s.V, s.r, dh.DSPARK_BF16, w2p, bp, stream.cuda_stream), 20)
        tok_b, conf_b, surv_b = torch.empty_like(tokens), torch.empty_like(conf), torch.empty_like(surv)
        bcalls = []
        for a in range(n_anch):
            c, _ = dh.prepare_head_sample(U[a : a + 1], Hh[a : a + 1], W["W1"], W["W2"], W["w_conf"], 0.0,
                                          X0[a : a + 1], tokens=tok_b[a : a + 1], conf=conf_b[a : a + 1],
                                          survival=surv_b[a : a + 1], workspace=ws, w2_bound=bound)
            bcalls.append(c)
        dh.workspace_status(ws)  # clear the path flags
        for c in bcalls[:10]:
            c()
        torch.cuda.synchronize()
        us_b = timed(lambda: [c() for c in bcalls], 1) / n_anch
        st_b, paths_b = dh.workspace_status(ws)
        same = int((tok_b == tokens).all(dim=1).sum().item())  # the serving step's tokens, same anchors
        # what the bounded call reads: U and h of the anchor, w_conf, the anchor's W1 row, the 64 sampled W2
        # rows and the bound (the few candidate rows the screen stages, at most 32 W1 and W2 rows, not counted)
        bytes_b = (s.gamma * s.V * 2 + s.gamma * s.H * 2 + (s.H + s.r) * 2 + s.r * 2 + 64 * s.r * 2
                   + 4 * dh.W2_BOUND_WORDS + 4 + s.gamma * 12)
        line["b1_w2bound"] = {
            "workload": f"B=1 gamma=7 V=151936 H=5120 r=256 bf16 greedy, the serving step's {n_anch} anchors back to "
                        "back with dspark_head_sample_w2bound: the largest W2 row norm computed once per weight load "
                        "(dspark_w2_bound) instead of a pass over W2 in every call",
            "us_per_call": round(us_b, 3), "positions_per_s": round(s.gamma / (us_b * 1e-6), 1),
            "w2_bound_us": round(bound_us, 2), "tokens_equal_to_plain_anchors": same, "anchors": n_anch,
            "give_up": st_b, "path_flags": paths_b,
            "roofline": hbm_roofline("dspark_head_sample_w2bound (bytes the call reads; W2 is not streamed)", bytes_b,
                                     us_b, None, None,
                                     timed_cold(lambda: bcalls[0](), 50) if scrub is not None else None),
        }
        del bcalls

    # ---------------- accept rate on the training-width workload ----------------
    if "accept" in legs:
        sa = synth.ACCEPT_TRAIN
        d, t = synth.accept_inputs(sa)
        D, T = to_dev(d, dev), to_dev(t, dev)
        del d, t
        acall, aout = dh.prepare_accept_rate(D, T)
        for _ in range(3):
            acall()
        torch.cuda.synchronize()
        a_us = timed(acall, 20)
        a_cold = timed_cold(acall, 10) if scrub is not None else None
        a_bytes = accept_call_bytes(sa.N, sa.V)
        gbs = a_bytes / (a_us * 1e-6) / 1e9
        line["accept_rate"] = {
            "value": round(gbs, 1), "unit": "GB/s",
            "workload": "analytic accept rate, 2048 positions x V=151936 bf16 draft/target logits",
            "us_per_call": round(a_us, 2), "positions_per_s": round(sa.N / (a_us * 1e-6), 1),
            "roofline": hbm_roofline("dspark_accept_rate (cluster kernel)", a_bytes, a_us,
                                     "accept_rate_cluster_2048x151936.md", ACCEPT_SOURCES, a_cold),
        }
        del D, T, aout

    # ---------------- rejection-sampling verify on the batched serving shape ----------------
    if "verify" in legs:
        sv = synth.VERIFY_B64
        vin = synth.verify_inputs(sv)
        vd = {k: to_dev(v, dev) for k, v in vin.items()}
        del vin
        vcall, vout = dh.prepare_verify(vd["d"], vd["t"], vd["x"], vd["u"], vd["G"])
        for _ in range(3):
            vcall()
        torch.cuda.synchronize()
        v_us = timed(vcall, 20)
        v_cold = timed_cold(vcall, 10) if scrub is not None else None
        n_acc = vout["n_accepted"].cpu().numpy()
        v_bytes = verify_call_bytes([sv.gamma] * sv.B, n_acc == sv.gamma, sv.V, sv.gamma)
        line["verify"] = {
            "workload": "rejection-sampling verify, B=64 requests x 7 drafted positions, V=151936 bf16 draft and "
                        "target logits, fp32 uniforms and Gumbel rows",
            "us_per_call": round(v_us, 2), "positions_per_s": round(sv.B * sv.gamma / (v_us * 1e-6), 1),
            "mean_accepted": round(float(n_acc.mean()), 3),
            "roofline": hbm_roofline("dspark_verify (2 launches; verify_stats reads every drafted row)", v_bytes,
                                     v_us, "verify_b64_vocab151936.md", VERIFY_SOURCES, v_cold),
        }
        del vd, vout

    # ---------------- batched Gumbel-max sampler (B=64) and the gated / RNN heads ----------------
    s3 = synth.SAMPLER_B64
    if legs & {"b64", "gated", "rnn"}:
        x3 = synth.sampler_batch(s3)
        d3 = {k: to_dev(x3[k], dev) for k in ("U", "h", "x0", "G")}
        del x3
        by3 = sampler_call_bytes(64, 7, s3.V, s3.H, s3.r) + 64 * 7 * s3.V * 4
        flops = 2.0 * 64 * s3.gamma * s3.V * s3.r
        # matrix-core bound with every byte read once: flops / (bytes at peak HBM)
        attain = flops / (by3 / (HBM_PEAK_GBS * 1e9)) / 1e12
    if "b64" in legs:
        ws3 = torch.zeros(dh.head_sample_workspace_size(64, 7, s3.V, s3.H, s3.r), dtype=torch.uint8, device=dev)
        c3, _ = dh.prepare_head_sample(d3["U"], d3["h"], W["W1"], W["W2"], W["w_conf"], 0.0, d3["x0"], d3["G"],
                                       workspace=ws3)
        for _ in range(3):
            c3()
        torch.cuda.synchronize()
        us3 = timed(c3, 20)
        cold3 = timed_cold(c3, 10) if scrub is not None else None
        tf = flops / (us3 * 1e-6) / 1e12
        line["b64"] = {
            "workload": "Markov-head block sampler, B=64 gamma=7 V=151936 H=5120 r=256 bf16, Gumbel-max with fp32 "
                        "noise",
            "us_per_call": round(us3, 2), "positions_per_s": round(64 * 7 / (us3 * 1e-6), 1),
            "mfma": {"tflops": round(tf, 2), "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                     "frac_of_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "attainable_tflops": round(attain, 1),
                     "attainable_frac_of_peak": round(attain / BF16_MFMA_PEAK_TFLOPS, 4),
                     "frac_of_attainable": round(tf / attain, 4),
                     "note": "bias GEMM 34.85 GFLOP per call; with W2, U and G each read once at 8 TB/s the matrix "
                             "cores cannot pass attainable_tflops"},
            "path_flags": dh.workspace_status(ws3)[1],
            "roofline": hbm_roofline("dspark_head_sample B=64 (one resident kernel)", by3, us3,
                                     "head_sample_resident_b64_vocab151936.md", SAMPLER_SOURCES, cold3),
        }
        del ws3
    if "gated" in legs:
        Wg3 = to_dev(synth.gate_weights(s3, 0.02), dev)
        cg, _ = dh.prepare_head_sample(d3["U"], d3["h"], W["W1"], W["W2"], W["w_conf"], 0.0, d3["x0"], d3["G"],
                                       Wg=Wg3)
        for _ in range(2):
            cg()
        torch.cuda.synchronize()
        usg = timed(cg, 10)
        g_cold = timed_cold(cg, 6) if scrub is not None else None
        byg = by3 + s3.r * (s3.H + s3.r) * 2
        line["gated_b64"] = {
            "workload": "gated Markov head, B=64 gamma=7 V=151936 H=5120 r=256 bf16, Gumbel-max with fp32 noise",
            "us_per_call": round(usg, 2), "positions_per_s": round(64 * 7 / (usg * 1e-6), 1),
            "roofline": hbm_roofline("dspark_head_sample_gated", byg, usg, "head_sample_gated_b64_vocab151936.md",
                                     SAMPLER_SOURCES, g_cold)}
        del Wg3
    if "rnn" in legs:
        Wr3 = tuple(to_dev(a, dev) for a in synth.rnn_weights(s3, 0.015))
        cr, _ = dh.prepare_head_sample(d3["U"], d3["h"], W["W1"], W["W2"], W["w_conf"], 0.0, d3["x0"], d3["G"],
                                       Wr=Wr3)
        for _ in range(2):
            cr()
        torch.cuda.synchronize()
        usr = timed(cr, 10)
        r_cold = timed_cold(cr, 6) if scrub is not None else None
        byr = by3 + 2 * s3.r * (2 * s3.r + s3.H) * 2
        line["rnn_b64"] = {
            "workload": "RNN head, B=64 gamma=7 V=151936 H=5120 r=256 bf16, Gumbel-max with fp32 noise",
            "us_per_call": round(usr, 2), "positions_per_s": round(64 * 7 / (usr * 1e-6), 1),
            "roofline": hbm_roofline("dspark_head_sample_rnn", byr, usr, "head_sample_rnn_b64_vocab151936.md",
                                     SAMPLER_SOURCES, r_cold)}
        del Wr3
    if legs & {"b64", "gated", "rnn"}:
        del d3

    # ---------------- prefix scheduler at training block width ----------------
    if "schedule" in legs:
        s5 = synth.SCHEDULE_TRAIN
        sch = {"workload": "prefix scheduler (Algorithm 1), B=256 requests x gamma=16, 4096-entry throughput "
                           "table; 'tokens': SPS(n) = n/(2+0.004n) as stated, 'steps': SPS(n) = 1/(2+0.004n)",
               "bound": "one workgroup: its vector ALUs and barriers"}
        for kind in ("tokens", "steps"):
            c5, o5 = dh.prepare_prefix_schedule(to_dev(synth.schedule_conf(s5), dev),
                                                to_dev(synth.sps_table(s5.n_sps, kind), dev), want_order=False)
            for _ in range(5):
                c5()
            torch.cuda.synchronize()
            sch[f"{kind}_us_per_call"] = round(timed(c5, 100), 2)
            sch[f"{kind}_n_selected"] = int(o5["n_selected"].item())
        line["schedule"] = sch

    # ---------------- teacher-forced block bias with the joint loss ----------------
    if "loss" in legs:
        s6 = synth.LOSS_TRAIN
        x6 = synth.loss_inputs(s6)
        d6 = {k: (to_dev(v, dev) if isinstance(v, np.ndarray) else v) for k, v in x6.items()}
        del x6
        c6, _ = dh.prepare_block_loss(d6["U"], d6["t"], d6["h"], d6["W1"], d6["W2"], d6["w_conf"], d6["b_conf"],
                                      d6["xp"], d6["y"])
        for _ in range(2):
            c6()
        torch.cuda.synchronize()
        us6 = timed(c6, 5)
        l_cold = timed_cold(c6, 3) if scrub is not None else None
        M6 = s6.N * s6.gamma
        by6 = (2 * M6 * s6.V * 2 + s6.V * s6.r * 2 + M6 * s6.r * 2 + M6 * s6.H * 2 + (s6.H + s6.r) * 2 + 8 * M6
               + 16 * M6 + 16)
        line["block_loss"] = {
            "workload": "teacher-forced block bias + joint loss (CE, L1, confidence BCE), 2048 positions "
                        "(128 anchors x block 16), V=151936 H=5120 r=256 bf16",
            "us_per_call": round(us6, 2), "positions_per_s": round(M6 / (us6 * 1e-6), 1),
            "mfma_tflops": round(2 * M6 * s6.V * s6.r / (us6 * 1e-6) / 1e12, 2),
            "roofline": hbm_roofline("dspark_block_loss", by6, us6, "block_loss_2048x151936.md", LOSS_SOURCES,
                                     l_cold)}
        del d6

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = 1 << 30

    # ---------------- CPU oracle on a bounded sample, and parity of those anchors ----------------
    if "cpu" in legs:
        from concurrent.futures import ThreadPoolExecutor

        import oracle

        ref = []
        tc0 = time.perf_counter()
        while len(ref) < len(host_batches) and (time.perf_counter() - tc0) < 10.0:
            x = host_batches[len(ref)]
            ref.append(oracle.head_sample(x["U"], x["h"], w["W1"], w["W2"], w["w_conf"], w["b_conf"], x["x0"]))
        t_one = (time.perf_counter() - tc0) / len(ref)
        conf_host = conf.cpu().numpy()
        tc1 = time.perf_counter()
        oracle.prefix_schedule(conf_host, sps_host)
        t_sched = time.perf_counter() - tc1
        # every host core: independent anchors on a thread pool (the C oracle
        # releases the interpreter lock while it runs)
        nthreads = os.cpu_count() or 1
        n_par = min(len(host_batches), 4 * nthreads)
        batch = host_batches[:n_par]
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            tp0 = time.perf_counter()
            list(ex.map(lambda x: oracle.head_sample(x["U"], x["h"], w["W1"], w["W2"], w["w_conf"], w["b_conf"],
                                                      x["x0"]), batch))
            t_par = (time.perf_counter() - tp0) / n_par
        cpu_step_1 = t_one * n_anch + t_sched
        cpu_step_n = t_par * n_anch + t_sched
        line["cpu_baseline"] = {
            "value": round(positions / cpu_step_n, 2), "unit": "draft positions/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"oracle sampler (fp64 C) on {n_par} of the {n_anch} anchors over {nthreads} threads "
                      f"({t_par * n_par:.1f} s) and on {len(ref)} anchors on one thread ({t_one * len(ref):.1f} s), "
                      f"each scaled to {n_anch} anchors, plus one oracle schedule of the {n_anch}x7 confidences "
                      f"({t_sched * 1e3:.1f} ms)",
            "single_thread_value": round(positions / cpu_step_1, 2),
            "nproc": nthreads, "cpu_model": cpu_model(),
        }
        # parity of the anchors the oracle computed against the GPU's tokens of
        # the timed steps: tokens up to the first difference, which must be a
        # near-tie (oracle margin < 1e-3)
        gtok = tokens.cpu().numpy()
        gconf = conf_host
        gsurv = surv.cpu().numpy()
        n_pos = n_eq = n_tie = n_bad = 0
        cerr = serr = 0.0
        for a, r in enumerate(ref):
            for k in range(s.gamma):
                n_pos += 1
                cerr = max(cerr, abs(float(gconf[a, k]) - r["conf"][0, k]))
                serr = max(serr, abs(float(gsurv[a, k]) - r["survival"][0, k]))
                if gtok[a, k] == r["tokens"][0, k]:
                    n_eq += 1
                    continue
                if r["margin"][0, k] < 1e-3:
                    n_tie += 1
                else:
                    n_bad += 1
                break
        line["parity"] = {"anchors": len(ref), "positions_compared": n_pos, "tokens_equal": n_eq,
                          "near_tie_stops": n_tie, "unexplained_mismatches": n_bad,
                          "conf_max_abs_err": float(f"{cerr:.3g}"), "survival_max_abs_err": float(f"{serr:.3g}"),
                          "rule": "per anchor, tokens compared in order up to the first difference, which must be "
                                  "an oracle near-tie (margin < 1e-3); conf and survival to 1e-4 over those steps"}

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
