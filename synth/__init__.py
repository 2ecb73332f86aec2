"""Seeded synthetic inputs for the DSpark draft-head hot path.

Random numbers only: nothing here computes any part of the method.  Both the
HIP path and the CPU oracle consume the host arrays produced here, so parity
does not depend on the generator.  Draws come from a counter-based SplitMix64
stream implemented in ``synth.c`` (see its header for the exact definition).

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bfloat16 bit
patterns (the upper half of an IEEE binary32).

Workload recipes (shapes, distributions, seeds) follow the synthetic
workloads of the DSpark draft-head configuration: hidden size 5120, Markov
rank 256, serving block 7 and training block 16 (dpshk.com article on the
Qwen3.8-27B-DSpark confidence head, section 3, config.json); the vocabulary
size 151936 is the Qwen3 tokenizer's.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# one master seed per workload, one tag per tensor
SEED_BASE = 0xD5A20000
TAG = {"W1": 1, "W2": 2, "U": 3, "h": 4, "w": 5, "x0": 6, "G": 7, "d": 8, "t": 9, "conf": 10, "sps": 11,
       "vd": 12, "vt": 13, "vtb": 14, "vx": 15, "vu": 16, "vG": 17, "Wg": 18, "Wrg": 19, "Wrc": 20,
       "lU": 21, "lt": 22, "lh": 23, "ly": 24, "lx": 25}


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "synth.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64, d, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_raw.restype = u64
        lib.synth_raw.argtypes = [u64, u64]
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            getattr(lib, name).argtypes = [u64, u64, i64, d, d, vp]
        lib.synth_affine_noise_bf16.argtypes = [u64, u64, i64, vp, d, d, d, vp]
        lib.synth_affine_noise_f32.argtypes = [u64, u64, i64, vp, d, d, d, vp]
        lib.synth_gumbel_f32.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform_int.argtypes = [u64, u64, i64, i64, i64, vp]
        lib.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
        lib.synth_logistic_conf.argtypes = [u64, i64, i64, d, d, d, vp]
        _lib = lib
    return _lib


def key(seed: int, tag: int) -> int:
    return int(_load().synth_key(seed & (2**64 - 1), tag & (2**64 - 1)))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(k: int, shape, mean: float, sd: float, dtype: str = "f32", start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, np.float32)
        _load().synth_normal_f32(k, start, n, mean, sd, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        _load().synth_normal_bf16(k, start, n, mean, sd, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def affine_noise(k: int, base: np.ndarray, scale: float, mean: float, sd: float, start: int = 0) -> np.ndarray:
    base = np.ascontiguousarray(base)
    out = np.empty_like(base)
    if base.dtype == np.uint16:
        _load().synth_affine_noise_bf16(k, start, base.size, _ptr(base), scale, mean, sd, _ptr(out))
    elif base.dtype == np.float32:
        _load().synth_affine_noise_f32(k, start, base.size, _ptr(base), scale, mean, sd, _ptr(out))
    else:
        raise ValueError(base.dtype)
    return out


def gumbel(k: int, shape, start: int = 0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_gumbel_f32(k, start, out.size, _ptr(out))
    return out


def uniform_int(k: int, shape, lo: int, hi: int, start: int = 0) -> np.ndarray:
    out = np.empty(shape, np.int32)
    _load().synth_uniform_int(k, start, out.size, lo, hi, _ptr(out))
    return out


def uniform(k: int, shape, start: int = 0) -> np.ndarray:
    out = np.empty(shape, np.float64)
    _load().synth_uniform_f64(k, start, out.size, _ptr(out))
    return out


def logistic_conf(k: int, B: int, gamma: int, mean: float, sd: float, slope: float) -> np.ndarray:
    out = np.empty((B, gamma), np.float32)
    _load().synth_logistic_conf(k, B, gamma, mean, sd, slope, _ptr(out))
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bit patterns, nearest-even (NaN kept quiet)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


# --------------------------------------------------------------------------
# Workload recipes
# --------------------------------------------------------------------------
@dataclass
class SamplerShape:
    B: int
    gamma: int
    V: int
    H: int
    r: int
    dtype: str  # "f32" or "bf16"
    w_sd: float  # sd of W1 and W2
    U_sd: float
    wc_sd: float  # sd of the confidence weight vector
    gumbel: bool
    seed: int


SAMPLER_TINY = SamplerShape(B=4, gamma=7, V=4096, H=256, r=32, dtype="f32", w_sd=0.05, U_sd=2.0, wc_sd=0.02,
                            gumbel=False, seed=SEED_BASE + 1)
SAMPLER_B1 = SamplerShape(B=1, gamma=7, V=151936, H=5120, r=256, dtype="bf16", w_sd=0.02, U_sd=3.0, wc_sd=0.01,
                          gumbel=False, seed=SEED_BASE + 2)
SAMPLER_B64 = SamplerShape(B=64, gamma=7, V=151936, H=5120, r=256, dtype="bf16", w_sd=0.02, U_sd=3.0, wc_sd=0.01,
                           gumbel=True, seed=SEED_BASE + 3)


def sampler_weights(s: SamplerShape, w_sd: float | None = None) -> dict:
    """Fixed weights: W1, W2 [V, r]; w_conf [H + r]; b_conf = 0."""
    sd = s.w_sd if w_sd is None else w_sd
    return {
        "W1": normal(key(s.seed, TAG["W1"]), (s.V, s.r), 0.0, sd, s.dtype),
        "W2": normal(key(s.seed, TAG["W2"]), (s.V, s.r), 0.0, sd, s.dtype),
        "w_conf": normal(key(s.seed, TAG["w"]), (s.H + s.r,), 0.0, s.wc_sd, s.dtype),
        "b_conf": 0.0,
    }


def gate_weights(s: SamplerShape, sd: float) -> np.ndarray:
    """Gate weights Wg [r, H + r] of the gated Markov head, N(0, sd), in the
    workload's dtype."""
    return normal(key(s.seed, TAG["Wg"]), (s.r, s.H + s.r), 0.0, sd, s.dtype)


def rnn_weights(s: SamplerShape, sd: float) -> tuple[np.ndarray, np.ndarray]:
    """Update-gate and candidate weights (Wrg, Wrc) [r, 2r + H] of the RNN head,
    N(0, sd), in the workload's dtype."""
    shape = (s.r, 2 * s.r + s.H)
    return (normal(key(s.seed, TAG["Wrg"]), shape, 0.0, sd, s.dtype),
            normal(key(s.seed, TAG["Wrc"]), shape, 0.0, sd, s.dtype))


def sampler_batch(s: SamplerShape, batch_id: int = 0, B: int | None = None) -> dict:
    """Per-call activations: U [B, gamma, V], h [B, gamma, H], anchors x0 [B],
    and, for Gumbel-max sampling, fp32 noise G [B, gamma, V].  Each batch id
    (an anchor index in the back-to-back B=1 workload) draws its own
    sub-streams; the weights stay fixed."""
    B = s.B if B is None else B
    tag = lambda t: key(s.seed, TAG[t] + (batch_id << 8))  # noqa: E731
    out = {
        "U": normal(tag("U"), (B, s.gamma, s.V), 0.0, s.U_sd, s.dtype),
        "h": normal(tag("h"), (B, s.gamma, s.H), 0.0, 1.0, s.dtype),
        "x0": uniform_int(tag("x0"), (B,), 0, s.V),
        "G": gumbel(tag("G"), (B, s.gamma, s.V)) if s.gumbel else None,
    }
    return out


@dataclass
class AcceptShape:
    N: int
    V: int
    dtype: str
    d_sd: float
    scale: float  # target = scale * draft + N(0, t_sd)
    t_sd: float
    seed: int


ACCEPT_TINY = AcceptShape(N=28, V=4096, dtype="f32", d_sd=2.0, scale=1.0, t_sd=0.5, seed=SEED_BASE + 1)
ACCEPT_TRAIN = AcceptShape(N=2048, V=151936, dtype="bf16", d_sd=3.0, scale=0.8, t_sd=1.5, seed=SEED_BASE + 4)


def accept_inputs(s: AcceptShape, N: int | None = None, row0: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Draft logits d [N, V] and target logits t = scale*d + noise, rows
    row0 .. row0+N-1 of the workload (so a sample of rows can be drawn
    without materialising the rest)."""
    N = s.N if N is None else N
    start = row0 * s.V
    d = normal(key(s.seed, TAG["d"]), (N, s.V), 0.0, s.d_sd, s.dtype, start=start)
    t = affine_noise(key(s.seed, TAG["t"]), d, s.scale, 0.0, s.t_sd, start=start)
    return d, t


@dataclass
class ScheduleShape:
    B: int
    gamma: int
    z_mean: float
    z_sd: float
    slope: float
    n_sps: int
    seed: int


SCHEDULE_TRAIN = ScheduleShape(B=256, gamma=16, z_mean=1.5, z_sd=1.5, slope=0.15, n_sps=4096, seed=SEED_BASE + 5)


def schedule_conf(s: ScheduleShape) -> np.ndarray:
    return logistic_conf(key(s.seed, TAG["conf"]), s.B, s.gamma, s.z_mean, s.z_sd, s.slope)


def sps_table(n_sps: int, kind: str = "tokens") -> np.ndarray:
    """Throughput curve as a table, sps[n-1] = SPS(n) for batch n = 1..n_sps.

    "tokens": SPS(n) = n / (2.0 + 0.004 n)   (the curve as stated)
    "steps":  SPS(n) = 1 / (2.0 + 0.004 n)   (the same step-time model read
              as verification steps per ms)
    """
    n = np.arange(1, n_sps + 1, dtype=np.float64)
    t = 2.0 + 0.004 * n
    if kind == "tokens":
        return n / t
    if kind == "steps":
        return 1.0 / t
    raise ValueError(kind)


@dataclass
class VerifyShape:
    """Rejection-sampling verification inputs: draft logits d [B, gamma, V],
    target logits t [B, gamma + 1, V] with t = scale*d + N(0, t_sd) at the
    drafted positions and N(0, d_sd) at the bonus position, drafted tokens
    uniform in [0, V), uniforms u [B, gamma] and Gumbel noise G [B, V]."""
    B: int
    gamma: int
    V: int
    dtype: str
    d_sd: float
    scale: float
    t_sd: float
    seed: int


# the batched serving shape: 64 requests, gamma 7, the full vocabulary, bf16
VERIFY_B64 = VerifyShape(B=64, gamma=7, V=151936, dtype="bf16", d_sd=3.0, scale=0.8, t_sd=1.5, seed=SEED_BASE + 6)
VERIFY_TINY = VerifyShape(B=4, gamma=7, V=4096, dtype="f32", d_sd=2.0, scale=1.0, t_sd=0.5, seed=SEED_BASE + 7)


def verify_inputs(s: VerifyShape, B: int | None = None) -> dict:
    B = s.B if B is None else B
    g, V = s.gamma, s.V
    d = normal(key(s.seed, TAG["vd"]), (B, g, V), 0.0, s.d_sd, s.dtype)
    t_draft = affine_noise(key(s.seed, TAG["vt"]), d, s.scale, 0.0, s.t_sd)
    t_bonus = normal(key(s.seed, TAG["vtb"]), (B, 1, V), 0.0, s.d_sd, s.dtype)
    t = np.ascontiguousarray(np.concatenate([t_draft, t_bonus], axis=1))
    return dict(
        d=d,
        t=t,
        x=uniform_int(key(s.seed, TAG["vx"]), (B, g), 0, V).astype(np.int32),
        # rounded to binary32 and kept below 1 (the accept test needs u < 1)
        u=np.minimum(uniform(key(s.seed, TAG["vu"]), (B, g)).astype(np.float32), np.float32(1 - 2**-24)),
        G=gumbel(key(s.seed, TAG["vG"]), (B, V)).astype(np.float32),
    )


@dataclass
class LossShape:
    """Teacher-forced block-loss inputs: N sequences' anchors x gamma block
    positions.  Draft backbone logits U ~ N(0, U_sd), target logits t =
    scale*U + N(0, t_sd), hidden states h ~ N(0, 1), targets y uniform in
    [0, V); the given previous tokens are the anchor (uniform) at the first
    position and the previous target after it (teacher forcing).  Weights as
    for the sampler: W1, W2 ~ N(0, w_sd), w_conf ~ N(0, wc_sd)."""
    N: int
    gamma: int
    V: int
    H: int
    r: int
    U_sd: float
    scale: float
    t_sd: float
    w_sd: float
    wc_sd: float
    seed: int


# 2048 training positions (8 sequences x 16 anchors x block 16) at the full vocabulary
LOSS_TRAIN = LossShape(N=128, gamma=16, V=151936, H=5120, r=256, U_sd=3.0, scale=0.8, t_sd=1.5, w_sd=0.02,
                       wc_sd=0.01, seed=SEED_BASE + 8)


def loss_inputs(s: LossShape, N: int | None = None) -> dict:
    N = s.N if N is None else N
    g, V = s.gamma, s.V
    U = normal(key(s.seed, TAG["lU"]), (N, g, V), 0.0, s.U_sd, "bf16")
    y = uniform_int(key(s.seed, TAG["ly"]), (N, g), 0, V).astype(np.int32)
    xp = np.empty((N, g), np.int32)
    xp[:, 0] = uniform_int(key(s.seed, TAG["lx"]), (N,), 0, V).astype(np.int32)
    xp[:, 1:] = y[:, :-1]
    return dict(
        U=U,
        t=affine_noise(key(s.seed, TAG["lt"]), U, s.scale, 0.0, s.t_sd),
        h=normal(key(s.seed, TAG["lh"]), (N, g, s.H), 0.0, 1.0, "bf16"),
        W1=normal(key(s.seed, TAG["W1"]), (V, s.r), 0.0, s.w_sd, "bf16"),
        W2=normal(key(s.seed, TAG["W2"]), (V, s.r), 0.0, s.w_sd, "bf16"),
        w_conf=normal(key(s.seed, TAG["w"]), (s.H + s.r,), 0.0, s.wc_sd, "bf16"),
        b_conf=0.0,
        xp=xp,
        y=y,
    )
