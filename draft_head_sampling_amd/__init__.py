"""Python binding of libdspark.so, the MI355X (gfx950) draft-head hot path.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/dspark.h``.  PyTorch supplies
device memory and the current stream, nothing else.  There is no fallback:
if the library is missing or no GPU is present, calls raise.

Entry points (same names as the C ABI):
  head_sample      Markov-head block sampler + confidence head + survival
  accept_rate      analytic accept rate 1 - 1/2 ||softmax(d) - softmax(t)||_1
  prefix_schedule  hardware-aware prefix scheduler (Algorithm 1)
  verify           rejection-sampling verification of a draft block
  block_loss       teacher-forced block bias with the joint training loss
  workspace_status give-up status and path flags of a workspace
  set_wait_limit   poll limit of the waits between workgroups

Environment: DSPARK_DEBUG=1 makes every call synchronise and raise on an
asynchronous HIP error or a wait that gave up.
"""
from __future__ import annotations

import ctypes
import os
from functools import partial

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")

DSPARK_F32, DSPARK_BF16 = 0, 1
_STATUS = {0: "ok", 1: "null argument", 2: "bad shape", 3: "bad dtype", 4: "workspace", 5: "HIP error"}

_lib = None


class DsparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status} ({_STATUS.get(status, '?')})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library, with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m draft_head_sampling_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    L.dspark_head_sample.restype = i32
    L.dspark_head_sample.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, sz, vp]
    L.dspark_accept_rate.restype = i32
    L.dspark_accept_rate.argtypes = [i64, i64, i32, vp, i64, vp, i64, vp, vp, sz, vp]
    L.dspark_prefix_schedule.restype = i32
    L.dspark_prefix_schedule.argtypes = [i64, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dspark_status_string.restype = ctypes.c_char_p
    L.dspark_status_string.argtypes = [i32]
    L.dspark_head_sample_workspace_size.restype = sz
    L.dspark_head_sample_gated.restype = i32
    L.dspark_head_sample_gated.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, sz, vp]
    L.dspark_head_sample_rnn.restype = i32
    L.dspark_head_sample_rnn.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, sz, vp]
    L.dspark_head_sample_rnn_workspace_size.restype = sz
    L.dspark_head_sample_rnn_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32]
    L.dspark_head_sample_gated_workspace_size.restype = sz
    L.dspark_head_sample_gated_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32]
    L.dspark_head_sample_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32]
    L.dspark_accept_rate_workspace_size.restype = sz
    L.dspark_accept_rate_workspace_size.argtypes = [i64, i64, i32]
    L.dspark_prefix_schedule_workspace_size.restype = sz
    L.dspark_prefix_schedule_workspace_size.argtypes = [i64, i64]
    L.dspark_verify.restype = i32
    L.dspark_verify.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dspark_verify_workspace_size.restype = sz
    L.dspark_verify_workspace_size.argtypes = [i64, i64, i64, i32]
    L.dspark_block_loss.restype = i32
    L.dspark_block_loss.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, f32,
                                    f32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dspark_block_loss_workspace_size.restype = sz
    L.dspark_block_loss_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32]
    L.dspark_head_sample_noalloc.restype = i32
    L.dspark_head_sample_noalloc.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp]
    L.dspark_head_sample_w2bound.restype = i32
    L.dspark_head_sample_w2bound.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, sz, vp]
    L.dspark_w2_bound.restype = i32
    L.dspark_w2_bound.argtypes = [i64, i64, i32, vp, vp, vp]
    L.dspark_workspace_status.restype = i32
    L.dspark_workspace_status.argtypes = [vp, sz, vp, vp]
    L.dspark_set_wait_limit.restype = i32
    L.dspark_set_wait_limit.argtypes = [i64, ctypes.POINTER(i64)]
    _lib = L
    return L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSPARK_F32
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, name, dtype=None, shape=None) -> int | None:
    return None if t is None else _dev(t, name, dtype, shape)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:  # zero-filled before first use, as the C ABI requires
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def _check(fn: str, status: int):
    if status != 0:
        raise DsparkError(fn, status)


class DsparkGaveUp(RuntimeError):
    """A bounded wait between workgroups ran out (the outputs of that call are
    unspecified; zero-fill the workspace before reusing it)."""


PATH_B1_REBUILD, PATH_B1_EXCHANGE, PATH_RESIDENT, PATH_ACCEPT_CLUSTER = 1, 2, 4, 8
PATH_B1_BOUND, PATH_B1_BOUND_STALE = 16, 32
W2_BOUND_WORDS = 8


def w2_bound(W2: torch.Tensor, stream=None) -> torch.Tensor:
    """dspark_w2_bound: the weights-only bound of the single-request screen
    for W2 [V, 256] bfloat16 (CUDA), as W2_BOUND_WORDS int32 words on W2's
    device; enqueued on the stream.  Pass it to prepare_head_sample(...,
    w2_bound=...) for as long as W2 is unchanged."""
    V, r = W2.shape
    out = torch.zeros(W2_BOUND_WORDS, dtype=torch.int32, device=W2.device)
    _check("dspark_w2_bound", lib().dspark_w2_bound(V, r, _dtype_code(W2), _dev(W2, "W2"), out.data_ptr(),
                                                    _stream(W2.device) if stream is None else stream))
    return out


def workspace_status(workspace: torch.Tensor) -> tuple[int, int]:
    """(give-up status, path flags) of a sampler / accept-rate / verify
    workspace, read in stream order (dspark_workspace_status); clears the
    path flags.  Synchronises the current stream to return host integers."""
    out = torch.zeros(2, dtype=torch.int32, device=workspace.device)
    _check("dspark_workspace_status",
           lib().dspark_workspace_status(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         out.data_ptr(), _stream(workspace.device)))
    st, paths = out.cpu().tolist()
    return int(st), int(paths) & 0xFFFFFFFF


def set_wait_limit(polls: int) -> int:
    """Process-wide poll limit of the waits between workgroups (negative =
    each kernel's default); returns the previous value (dspark_set_wait_limit)."""
    prev = ctypes.c_int64(0)
    _check("dspark_set_wait_limit", lib().dspark_set_wait_limit(int(polls), ctypes.byref(prev)))
    return int(prev.value)


def _debug() -> bool:
    return os.environ.get("DSPARK_DEBUG", "") == "1"


def _caller(name: str, fn, ws):
    """The enqueue function of a prepared call.  With DSPARK_DEBUG=1 every
    call synchronises, surfaces asynchronous HIP errors, and raises
    DsparkGaveUp when the workspace's give-up word is set."""
    if not _debug():
        return lambda: _check(name, fn())

    def call():
        _check(name, fn())
        torch.cuda.synchronize()
        if ws is not None and name != "dspark_block_loss":
            st, _ = workspace_status(ws)
            if st:
                raise DsparkGaveUp(f"{name}: a wait between workgroups gave up (were other kernels holding "
                                   "compute units?); outputs are unspecified; zero-fill the workspace")
    return call


def head_sample_workspace_size(B, gamma, V, H, r, dtype=DSPARK_BF16) -> int:
    return int(lib().dspark_head_sample_workspace_size(B, gamma, V, H, r, dtype))


def prepare_head_sample(U, h, W1, W2, w_conf, b_conf, x0, gumbel=None, force=None, *, tokens=None, conf=None,
                        survival=None, logits_out=None, bias_out=None, workspace=None, stream=None, Wg=None, Wr=None,
                        w2_bound=None):
    """Validate once and return (call, outputs): ``call()`` enqueues
    dspark_head_sample (or, with gate weights Wg [r, H + r], the gated head
    dspark_head_sample_gated; with Wr = (Wrg, Wrc), each [r, 2r + H], the RNN
    head dspark_head_sample_rnn; with the words of w2_bound(W2),
    dspark_head_sample_w2bound) on the stream with these exact buffers."""
    B, gamma, V = U.shape
    r = W1.shape[1]
    H = h.shape[2] if h is not None else 0
    dt = _dtype_code(U)
    dev = U.device
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev) if tokens is None else tokens
    conf = torch.empty((B, gamma), dtype=torch.float32, device=dev) if conf is None else conf
    survival = torch.empty((B, gamma), dtype=torch.float32, device=dev) if survival is None else survival
    args = (
        B, gamma, V, H, r, dt,
        _dev(U, "U", U.dtype, (B, gamma, V)),
        _opt(h, "h", U.dtype, (B, gamma, H)),
        _dev(W1, "W1", U.dtype, (V, r)),
        _dev(W2, "W2", U.dtype, (V, r)),
        _dev(w_conf, "w_conf", U.dtype, (H + r,)),
        float(b_conf),
        _dev(x0, "x0", torch.int32, (B,)),
        _opt(gumbel, "gumbel", torch.float32, (B, gamma, V)),
        _opt(force, "force", torch.int32, (B, gamma)),
        _dev(tokens, "tokens", torch.int32, (B, gamma)),
        _dev(conf, "conf", torch.float32, (B, gamma)),
        _dev(survival, "survival", torch.float32, (B, gamma)),
        _opt(logits_out, "logits_out", torch.float32, (B, gamma, V)),
        _opt(bias_out, "bias_out", torch.float32, (B, gamma, V)),
    )
    st = _stream(dev) if stream is None else stream
    if Wg is not None and Wr is not None:
        raise ValueError("Wg (gated head) and Wr (RNN head) are exclusive")
    if w2_bound is not None and (Wg is not None or Wr is not None):
        raise ValueError("w2_bound applies to the Markov head only")
    if Wr is not None:
        rargs = args[:11] + (_dev(Wr[0], "Wrg", U.dtype, (r, 2 * r + H)),
                             _dev(Wr[1], "Wrc", U.dtype, (r, 2 * r + H))) + args[11:]
        ws, wsb = _workspace(int(lib().dspark_head_sample_rnn_workspace_size(B, gamma, V, H, r, dt)), dev,
                             workspace)
        fn = partial(lib().dspark_head_sample_rnn, *rargs, None if ws is None else ws.data_ptr(), wsb, st)
        name = "dspark_head_sample_rnn"
    elif Wg is None and w2_bound is not None:
        ws, wsb = _workspace(head_sample_workspace_size(B, gamma, V, H, r, dt), dev, workspace)
        bw = _dev(w2_bound, "w2_bound", torch.int32, (W2_BOUND_WORDS,))
        fn = partial(lib().dspark_head_sample_w2bound, *args, bw, None if ws is None else ws.data_ptr(), wsb, st)
        name = "dspark_head_sample_w2bound"
    elif Wg is None:
        ws, wsb = _workspace(head_sample_workspace_size(B, gamma, V, H, r, dt), dev, workspace)
        fn = partial(lib().dspark_head_sample, *args, None if ws is None else ws.data_ptr(), wsb, st)
        name = "dspark_head_sample"
    else:
        gargs = args[:11] + (_dev(Wg, "Wg", U.dtype, (r, H + r)),) + args[11:]
        ws, wsb = _workspace(int(lib().dspark_head_sample_gated_workspace_size(B, gamma, V, H, r, dt)), dev,
                             workspace)
        fn = partial(lib().dspark_head_sample_gated, *gargs, None if ws is None else ws.data_ptr(), wsb, st)
        name = "dspark_head_sample_gated"
    outs = {"tokens": tokens, "conf": conf, "survival": survival, "_workspace": ws}
    if logits_out is not None:
        outs["logits"] = logits_out
    if bias_out is not None:
        outs["bias"] = bias_out
    return _caller(name, fn, ws), outs


def head_sample(U, h, W1, W2, w_conf, b_conf, x0, gumbel=None, force=None, *, want_logits=False, workspace=None,
                Wg=None, Wr=None):
    """Sample one draft block per request.

    U [B, gamma, V], h [B, gamma, H], W1/W2 [V, r], w_conf [H + r]: float32 or
    bfloat16 CUDA tensors of one dtype; x0 [B] int32; gumbel [B, gamma, V]
    float32 or None (greedy); force [B, gamma] int32 (-1 = sample) or None;
    Wg [r, H + r] (same dtype) selects the gated Markov head, Wr = (Wrg,
    Wrc), each [r, 2r + H], the RNN head.
    Returns dict(tokens [B, gamma] int32, conf, survival [B, gamma] float32
    [, logits, bias [B, gamma, V] float32 when want_logits]).
    """
    lo = bo = None
    if want_logits:
        lo = torch.empty(U.shape, dtype=torch.float32, device=U.device)
        bo = torch.empty(U.shape, dtype=torch.float32, device=U.device)
    call, outs = prepare_head_sample(U, h, W1, W2, w_conf, b_conf, x0, gumbel, force, logits_out=lo, bias_out=bo,
                                     workspace=workspace, Wg=Wg, Wr=Wr)
    call()
    outs.pop("_workspace")
    return outs


def head_sample_noalloc(U, h, W1, W2, w_conf, b_conf, x0, gumbel=None, force=None):
    """dspark_head_sample_noalloc: the sampler on the library's static
    per-GPU scratch array (no workspace argument, nothing allocated by the
    library).  Same arguments and outputs as head_sample (no stored logits)."""
    B, gamma, V = U.shape
    r = W1.shape[1]
    H = h.shape[2] if h is not None else 0
    dev = U.device
    outs = {"tokens": torch.empty((B, gamma), dtype=torch.int32, device=dev),
            "conf": torch.empty((B, gamma), dtype=torch.float32, device=dev),
            "survival": torch.empty((B, gamma), dtype=torch.float32, device=dev)}
    st = lib().dspark_head_sample_noalloc(
        B, gamma, V, H, r, _dtype_code(U), _dev(U, "U", U.dtype, (B, gamma, V)), _opt(h, "h", U.dtype, (B, gamma, H)),
        _dev(W1, "W1", U.dtype, (V, r)), _dev(W2, "W2", U.dtype, (V, r)), _dev(w_conf, "w_conf", U.dtype, (H + r,)),
        float(b_conf), _dev(x0, "x0", torch.int32, (B,)), _opt(gumbel, "gumbel", torch.float32, (B, gamma, V)),
        _opt(force, "force", torch.int32, (B, gamma)), _dev(outs["tokens"], "tokens"), _dev(outs["conf"], "conf"),
        _dev(outs["survival"], "survival"), None, None, _stream(dev))
    _check("dspark_head_sample_noalloc", st)
    return outs


def prepare_accept_rate(draft, target, V=None, *, out=None, workspace=None, stream=None):
    N, ldd = draft.shape
    ldt = target.shape[1]
    V = ldd if V is None else V
    dt = _dtype_code(draft)
    dev = draft.device
    if target.shape[0] != N:
        raise ValueError("draft and target need the same number of rows")
    out = torch.empty(N, dtype=torch.float32, device=dev) if out is None else out
    ws, wsb = _workspace(int(lib().dspark_accept_rate_workspace_size(N, V, dt)), dev, workspace)
    args = (N, V, dt, _dev(draft, "draft", draft.dtype), ldd, _dev(target, "target", draft.dtype), ldt,
            _dev(out, "accept_rate", torch.float32, (N,)), None if ws is None else ws.data_ptr(), wsb,
            _stream(dev) if stream is None else stream)
    fn = partial(lib().dspark_accept_rate, *args)
    return _caller("dspark_accept_rate", fn, ws), {"accept_rate": out, "_workspace": ws}


def accept_rate(draft, target, V=None, *, workspace=None):
    """c*_n = 1 - 1/2 ||softmax(draft_n[:V]) - softmax(target_n[:V])||_1.

    draft [N, ld_d], target [N, ld_t]: float32 or bfloat16 CUDA tensors (the
    row stride may exceed V).  Returns float32 [N]."""
    call, outs = prepare_accept_rate(draft, target, V, workspace=workspace)
    call()
    return outs["accept_rate"]


def prepare_prefix_schedule(conf, sps, *, want_order=True, workspace=None, stream=None):
    B, gamma = conf.shape
    dev = conf.device
    n_sps = sps.shape[0]
    outs = {
        "prefix_len": torch.empty(B, dtype=torch.int32, device=dev),
        "survival": torch.empty((B, gamma), dtype=torch.float32, device=dev),
        "order": torch.empty(B * gamma, dtype=torch.int32, device=dev) if want_order else None,
        "theta": torch.empty(1, dtype=torch.float64, device=dev),
        "n_selected": torch.empty(1, dtype=torch.int32, device=dev),
    }
    ws, wsb = _workspace(int(lib().dspark_prefix_schedule_workspace_size(B, gamma)), dev, workspace)
    args = (B, gamma, _dev(conf, "conf", torch.float32, (B, gamma)), _dev(sps, "sps", torch.float64, (n_sps,)), n_sps,
            _dev(outs["prefix_len"], "prefix_len"), _dev(outs["survival"], "survival"),
            _opt(outs["order"], "order"), _dev(outs["theta"], "theta"), _dev(outs["n_selected"], "n_selected"),
            None if ws is None else ws.data_ptr(), wsb, _stream(dev) if stream is None else stream)
    fn = partial(lib().dspark_prefix_schedule, *args)
    outs["_workspace"] = ws
    return _caller("dspark_prefix_schedule", fn, ws), outs


def prefix_schedule(conf, sps, *, want_order=True, workspace=None):
    """Algorithm 1 on conf [B, gamma] float32 and sps [n_sps] float64 (CUDA).

    Returns dict(prefix_len [B] int32, survival [B, gamma] float32,
    order [B*gamma] int32, theta [1] float64, n_selected [1] int32)."""
    call, outs = prepare_prefix_schedule(conf, sps, want_order=want_order, workspace=workspace)
    call()
    outs.pop("_workspace")
    return outs


def prepare_verify(draft, target, draft_tokens, uniforms, gumbel, n_draft=None, *, want_accept_prob=False,
                   workspace=None, stream=None):
    B, gp1, V = target.shape
    gamma = gp1 - 1
    dt = _dtype_code(target)
    dev = target.device
    outs = {
        "n_accepted": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "accept_prob": torch.empty((B, gamma), dtype=torch.float32, device=dev) if want_accept_prob else None,
    }
    ws, wsb = _workspace(int(lib().dspark_verify_workspace_size(B, gamma, V, dt)), dev, workspace)
    args = (B, gamma, V, dt, _dev(draft, "draft", target.dtype, (B, gamma, V)), _dev(target, "target"),
            _dev(draft_tokens, "draft_tokens", torch.int32, (B, gamma)), _opt(n_draft, "n_draft", torch.int32, (B,)),
            _dev(uniforms, "uniforms", torch.float32, (B, gamma)), _dev(gumbel, "gumbel", torch.float32, (B, V)),
            _dev(outs["n_accepted"], "n_accepted"), _dev(outs["next_token"], "next_token"),
            _opt(outs["accept_prob"], "accept_prob"), None if ws is None else ws.data_ptr(), wsb,
            _stream(dev) if stream is None else stream)
    fn = partial(lib().dspark_verify, *args)
    outs["_workspace"] = ws
    return _caller("dspark_verify", fn, ws), outs


def verify(draft, target, draft_tokens, uniforms, gumbel, n_draft=None, *, want_accept_prob=False, workspace=None):
    """Rejection-sampling verification of one draft block per request.

    draft [B, gamma, V] and target [B, gamma + 1, V] logits (float32 or
    bfloat16), draft_tokens [B, gamma] int32, uniforms [B, gamma] float32 in
    [0, 1), gumbel [B, V] float32, n_draft [B] int32 or None (= gamma).
    Returns dict(n_accepted [B], next_token [B], accept_prob [B, gamma] or
    None)."""
    call, outs = prepare_verify(draft, target, draft_tokens, uniforms, gumbel, n_draft,
                                want_accept_prob=want_accept_prob, workspace=workspace)
    call()
    outs.pop("_workspace")
    return outs


def prepare_block_loss(U, t, h, W1, W2, w_conf, b_conf, xp, y, mask=None, *, decay=4.0, a_ce=0.1, a_l1=0.9,
                       a_conf=1.0, workspace=None, stream=None):
    """Validate once and return (call, outputs) for dspark_block_loss: the
    teacher-forced block bias with the joint loss over U, t [N, gamma, V],
    h [N, gamma, H], W1, W2 [V, 256], w_conf [H + 256] (bfloat16), xp, y
    [N, gamma] int32 and mask [N, gamma] float32 or None."""
    N, gamma, V = U.shape
    r = W1.shape[1]
    H = h.shape[2] if h is not None else 0
    dt = _dtype_code(U)
    dev = U.device
    outs = {k: torch.empty((N, gamma), dtype=torch.float32, device=dev) for k in ("ce", "l1", "conf", "bce")}
    outs["loss"] = torch.empty(4, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(int(lib().dspark_block_loss_workspace_size(N, gamma, V, H, r, dt)), dev, workspace)
    args = (N, gamma, V, H, r, dt, _dev(U, "U", U.dtype, (N, gamma, V)), _dev(t, "t", U.dtype, (N, gamma, V)),
            _opt(h, "h", U.dtype, (N, gamma, H)), _dev(W1, "W1", U.dtype, (V, r)), _dev(W2, "W2", U.dtype, (V, r)),
            _dev(w_conf, "w_conf", U.dtype, (H + r,)), float(b_conf), _dev(xp, "xp", torch.int32, (N, gamma)),
            _dev(y, "y", torch.int32, (N, gamma)), _opt(mask, "mask", torch.float32, (N, gamma)), float(decay),
            float(a_ce), float(a_l1), float(a_conf), _dev(outs["ce"], "ce"), _dev(outs["l1"], "l1"),
            _dev(outs["conf"], "conf"), _dev(outs["bce"], "bce"), _dev(outs["loss"], "loss"),
            None if ws is None else ws.data_ptr(), wsb, _stream(dev) if stream is None else stream)
    fn = partial(lib().dspark_block_loss, *args)
    outs["_workspace"] = ws
    return _caller("dspark_block_loss", fn, ws), outs


def block_loss(U, t, h, W1, W2, w_conf, b_conf, xp, y, mask=None, *, decay=4.0, a_ce=0.1, a_l1=0.9, a_conf=1.0,
               workspace=None):
    """Teacher-forced block bias with the joint loss.  Returns dict(ce, l1,
    conf, bce [N, gamma], loss [4] = (L, L_ce, L_l1, L_conf))."""
    call, outs = prepare_block_loss(U, t, h, W1, W2, w_conf, b_conf, xp, y, mask, decay=decay, a_ce=a_ce,
                                    a_l1=a_l1, a_conf=a_conf, workspace=workspace)
    call()
    outs.pop("_workspace")
    return outs
