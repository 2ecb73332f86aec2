"""CPU oracle for the DSpark draft-head hot path -- test infrastructure.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never calls it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, single-threaded); this
module only compiles it with gcc and marshals numpy arrays.  Each function
cites the passage of the pages it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSPARK_ORACLE_SANITIZE=1 selects a build with AddressSanitizer and
# UndefinedBehaviorSanitizer (CPU only; the process needs libasan preloaded,
# see run_sanitized.sh beside this file).
_SANITIZE = os.environ.get("DSPARK_ORACLE_SANITIZE", "") == "1"
_SO = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True, sanitize: bool | None = None) -> str:
    san = _SANITIZE if sanitize is None else sanitize
    so = os.path.join(_HERE, "liboracle_san.so" if san else "liboracle.so")
    if force or not os.path.exists(so):
        tmp = so + ".tmp"
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined"] if san else ["-O2"]
        subprocess.check_call(["gcc", *flags, "-fPIC", "-shared", "-o", tmp, os.path.join(_HERE, "oracle.c"), "-lm"])
        os.replace(tmp, so)
    return so


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, vp, d = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_head_sample.restype = ctypes.c_int
        lib.oracle_head_sample.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, d,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_accept_rate.restype = ctypes.c_int
        lib.oracle_accept_rate.argtypes = [i64, i64, ctypes.c_int, vp, i64, vp, i64, vp, vp]
        lib.oracle_prefix_schedule.restype = ctypes.c_int
        lib.oracle_prefix_schedule.argtypes = [i64, i64, vp, vp, i64, vp, vp, vp, vp, vp]
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_verify.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_block_loss.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, d, vp, vp,
                                          vp, d, d, d, d, vp, vp, vp, vp, vp]
        _lib = lib
    return _lib


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or bfloat16 bit patterns (uint16), got {a.dtype}")


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def head_sample(U, h, W1, W2, w_conf, b_conf, x0, gumbel=None, force=None, want_logits=False, Wg=None, Wr=None):
    """Markov-head block sampler + confidence head + survival (fp64).

    U [B, gamma, V], h [B, gamma, H], W1/W2 [V, r], w_conf [H + r] share one
    dtype (float32, or uint16 bfloat16 bits).  x0 [B] int32, gumbel
    [B, gamma, V] float32 or None, force [B, gamma] int32 (-1 = sample) or
    None.  Wg [r, H + r] (same dtype) selects the gated Markov head; Wr =
    (Wrg, Wrc), each [r, 2r + H], the RNN head.  Returns a dict of tokens,
    conf, survival, margin (and logits, bias when ``want_logits``).
    """
    U, h, W1, W2, w_conf = (np.ascontiguousarray(a) for a in (U, h, W1, W2, w_conf))
    dt = _dtype_of(U)
    for a in (h, W1, W2, w_conf):
        assert _dtype_of(a) == dt
    B, gamma, V = U.shape
    H = h.shape[2]
    r = W1.shape[1]
    assert h.shape[:2] == (B, gamma) and W1.shape == (V, r) and W2.shape == (V, r) and w_conf.shape == (H + r,)
    x0 = np.ascontiguousarray(x0, dtype=np.int32)
    if gumbel is not None:
        gumbel = np.ascontiguousarray(gumbel, dtype=np.float32)
        assert gumbel.shape == U.shape
    if force is not None:
        force = np.ascontiguousarray(force, dtype=np.int32)
        assert force.shape == (B, gamma)
    if Wg is not None:
        Wg = np.ascontiguousarray(Wg)
        assert _dtype_of(Wg) == dt and Wg.shape == (r, H + r)
    Wrg = Wrc = None
    if Wr is not None:
        Wrg, Wrc = (np.ascontiguousarray(a) for a in Wr)
        for a in (Wrg, Wrc):
            assert _dtype_of(a) == dt and a.shape == (r, 2 * r + H)
    out = {
        "tokens": np.empty((B, gamma), np.int32),
        "conf": np.empty((B, gamma), np.float64),
        "survival": np.empty((B, gamma), np.float64),
        "margin": np.empty((B, gamma), np.float64),
    }
    if want_logits:
        out["logits"] = np.empty((B, gamma, V), np.float64)
        out["bias"] = np.empty((B, gamma, V), np.float64)
    rc = _load().oracle_head_sample(B, gamma, V, H, r, dt, _p(U), _p(h), _p(W1), _p(W2), _p(w_conf),
                                    float(b_conf), _p(x0), _p(gumbel), _p(force), _p(out["tokens"]),
                                    _p(out["conf"]), _p(out["survival"]), _p(out["margin"]),
                                    _p(out.get("logits")), _p(out.get("bias")), _p(Wg), _p(Wrg), _p(Wrc))
    if rc != 0:
        raise ValueError(f"oracle_head_sample failed ({rc}): token id out of range")
    return out


def accept_rate(d, t, V=None, with_summin=False):
    """c*_n = 1 - 1/2 ||softmax(d_n) - softmax(t_n)||_1 per row (fp64).

    d, t [N, ld] float32 or bfloat16 bits; the first V columns form a row."""
    d = np.ascontiguousarray(d)
    t = np.ascontiguousarray(t)
    dt = _dtype_of(d)
    assert _dtype_of(t) == dt
    N = d.shape[0]
    assert t.shape[0] == N
    V = d.shape[1] if V is None else V
    cs = np.empty(N, np.float64)
    sm = np.empty(N, np.float64) if with_summin else None
    _load().oracle_accept_rate(N, V, dt, _p(d), d.shape[1], _p(t), t.shape[1], _p(cs), _p(sm))
    return (cs, sm) if with_summin else cs


def prefix_schedule(conf, sps):
    """Algorithm 1 on conf [B, gamma] float32 and sps [n_sps] float64.

    Returns dict(prefix_len [B] int32, survival [B, gamma] float32,
    order [B*gamma] int32, theta float, n_selected int)."""
    conf = np.ascontiguousarray(conf, dtype=np.float32)
    sps = np.ascontiguousarray(sps, dtype=np.float64)
    B, gamma = conf.shape
    out = {
        "prefix_len": np.empty(B, np.int32),
        "survival": np.empty((B, gamma), np.float32),
        "order": np.empty(B * gamma, np.int32),
    }
    th = np.empty(1, np.float64)
    ns = np.empty(1, np.int64)
    rc = _load().oracle_prefix_schedule(B, gamma, _p(conf), _p(sps), sps.shape[0], _p(out["prefix_len"]),
                                        _p(out["survival"]), _p(out["order"]), _p(th), _p(ns))
    if rc != 0:
        raise ValueError("oracle_prefix_schedule: need B >= 1 and a table of at least B entries")
    out["theta"] = float(th[0])
    out["n_selected"] = int(ns[0])
    return out


def verify(d, t, x, u, G, n_draft=None):
    """Rejection-sampling verification of one draft block per request (fp64).

    d [B, gamma, V] and t [B, gamma + 1, V] float32 or bfloat16 bits, x
    [B, gamma] int32 drafted tokens, u [B, gamma] float32 uniforms in [0, 1),
    G [B, V] float32 Gumbel noise, n_draft [B] int32 or None (= gamma).
    Returns dict(n_acc, next_token, accept_prob [B, gamma], margin,
    sample_pos, residual)."""
    d = np.ascontiguousarray(d)
    t = np.ascontiguousarray(t)
    dt = _dtype_of(d)
    assert _dtype_of(t) == dt
    B, gamma, V = d.shape
    assert t.shape == (B, gamma + 1, V)
    x = np.ascontiguousarray(x, dtype=np.int32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    G = np.ascontiguousarray(G, dtype=np.float32)
    assert x.shape == (B, gamma) and u.shape == (B, gamma) and G.shape == (B, V)
    if n_draft is not None:
        n_draft = np.ascontiguousarray(n_draft, dtype=np.int32)
        assert n_draft.shape == (B,)
    out = {
        "n_acc": np.empty(B, np.int32),
        "next_token": np.empty(B, np.int32),
        "accept_prob": np.empty((B, gamma), np.float64),
        "margin": np.empty(B, np.float64),
        "sample_pos": np.empty(B, np.int32),
        "residual": np.empty(B, np.int32),
    }
    _load().oracle_verify(B, gamma, V, dt, _p(d), _p(t), _p(x), _p(n_draft), _p(u), _p(G), _p(out["n_acc"]),
                          _p(out["next_token"]), _p(out["accept_prob"]), _p(out["margin"]), _p(out["sample_pos"]),
                          _p(out["residual"]))
    return out


def block_loss(U, t, h, W1, W2, w_conf, b_conf, xp, y, mask=None, decay=4.0, a_ce=0.1, a_l1=0.9, a_conf=1.0):
    """Teacher-forced block bias with the joint loss (fp64).

    U, t [N, gamma, V], h [N, gamma, H], W1, W2 [V, r], w_conf [H + r] in
    float32 or bfloat16 bits; xp, y [N, gamma] int32 (given previous tokens,
    target ids); mask [N, gamma] float32 or None.  Returns dict(ce, l1, conf,
    bce [N, gamma], loss, L_ce, L_l1, L_conf)."""
    U, t, h, W1, W2, w_conf = (np.ascontiguousarray(a) for a in (U, t, h, W1, W2, w_conf))
    dt = _dtype_of(U)
    N, gamma, V = U.shape
    H = h.shape[2]
    r = W1.shape[1]
    assert t.shape == U.shape and W2.shape == (V, r) and w_conf.shape == (H + r,)
    xp = np.ascontiguousarray(xp, dtype=np.int32)
    y = np.ascontiguousarray(y, dtype=np.int32)
    mask = None if mask is None else np.ascontiguousarray(mask, dtype=np.float32)
    out = {k: np.empty((N, gamma), np.float64) for k in ("ce", "l1", "conf", "bce")}
    loss = np.empty(4, np.float64)
    rc = _load().oracle_block_loss(N, gamma, V, H, r, dt, _p(U), _p(t), _p(h), _p(W1), _p(W2), _p(w_conf),
                                   float(b_conf), _p(xp), _p(y), _p(mask), float(decay), float(a_ce), float(a_l1),
                                   float(a_conf), _p(out["ce"]), _p(out["l1"]), _p(out["conf"]), _p(out["bce"]),
                                   _p(loss))
    if rc != 0:
        raise MemoryError("oracle_block_loss: allocation failed")
    out.update(loss=float(loss[0]), L_ce=float(loss[1]), L_l1=float(loss[2]), L_conf=float(loss[3]))
    return out
