"""The C ABI without a GPU: the library loads, exports every function that
include/dspark.h declares, answers workspace queries, and rejects bad
arguments on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import draft_head_sampling_amd as dh

    if not os.path.exists(dh.LIB_PATH):
        from draft_head_sampling_amd import build

        build.build()
    return dh.lib()


def test_exports_every_declared_function(L):
    hdr = open(os.path.join(ROOT, "include", "dspark.h")).read()
    names = set(re.findall(r"^\s*(?:dspark_status_t|size_t|const char\*)\s+(dspark_\w+)\s*\(", hdr, re.M))
    assert {"dspark_head_sample", "dspark_accept_rate", "dspark_prefix_schedule"} <= names
    for n in names:
        assert hasattr(L, n), n
    # nothing else is exported under the dspark_ prefix
    import subprocess

    syms = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "draft_head_sampling_amd",
                                                                       "libdspark.so")],
                          capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dspark_\w+)", syms))
    assert exported == names


def test_status_strings(L):
    for s in range(6):
        assert L.dspark_status_string(s)


OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x1000  # never dereferenced: every case below fails or returns before any launch


def _hs(L, B=1, gamma=7, V=100, H=8, r=16, dtype=1, U=FAKE, h=FAKE, W1=FAKE, W2=FAKE, w=FAKE, x0=FAKE, tokens=FAKE,
        conf=FAKE, surv=FAKE, ws=None, wsb=0):
    return L.dspark_head_sample(B, gamma, V, H, r, dtype, U, h, W1, W2, w, 0.0, x0, None, None, tokens, conf, surv,
                                None, None, ws, wsb, None)


def test_head_sample_validation(L):
    assert _hs(L, dtype=2) == BAD_DTYPE
    assert _hs(L, B=-1) == BAD_SHAPE
    assert _hs(L, V=0) == BAD_SHAPE
    assert _hs(L, r=0) == BAD_SHAPE
    assert _hs(L, r=4096) == BAD_SHAPE
    assert _hs(L, H=-3) == BAD_SHAPE
    assert _hs(L, V=2**31) == BAD_SHAPE
    assert _hs(L, B=2**40, gamma=2**30) == BAD_SHAPE
    assert _hs(L, B=0) == OK and _hs(L, gamma=0) == OK  # empty: nothing enqueued
    need = L.dspark_head_sample_workspace_size(1, 7, 100, 8, 16, 1)
    assert need > 0
    assert _hs(L) == WORKSPACE  # no workspace
    assert _hs(L, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _hs(L, ws=FAKE + 8, wsb=need) == WORKSPACE  # misaligned
    assert _hs(L, ws=FAKE, wsb=need, U=None) == NULL_ARG
    assert _hs(L, ws=FAKE, wsb=need, x0=None) == NULL_ARG
    assert _hs(L, ws=FAKE, wsb=need, h=None) == NULL_ARG
    assert _hs(L, ws=FAKE, wsb=need, tokens=None) == NULL_ARG


def test_accept_rate_validation(L):
    f = L.dspark_accept_rate
    assert f(4, 10, 7, FAKE, 10, FAKE, 10, FAKE, None, 0, None) == BAD_DTYPE
    assert f(4, 10, 0, FAKE, 9, FAKE, 10, FAKE, None, 0, None) == BAD_SHAPE
    assert f(4, 10, 0, FAKE, 10, FAKE, 9, FAKE, None, 0, None) == BAD_SHAPE
    assert f(-1, 10, 0, FAKE, 10, FAKE, 10, FAKE, None, 0, None) == BAD_SHAPE
    assert f(4, 0, 0, FAKE, 10, FAKE, 10, FAKE, None, 0, None) == BAD_SHAPE
    assert f(0, 10, 0, None, 10, None, 10, None, None, 0, None) == OK
    need = L.dspark_accept_rate_workspace_size(4, 10, 0)
    ws = FAKE if need else None
    assert f(4, 10, 0, None, 10, FAKE, 10, FAKE, ws, need, None) == NULL_ARG
    assert f(4, 10, 0, FAKE, 10, FAKE, 10, None, ws, need, None) == NULL_ARG


def test_prefix_schedule_validation(L):
    f = L.dspark_prefix_schedule
    assert f(0, 4, FAKE, FAKE, 10, FAKE, None, None, None, None, None, 0, None) == BAD_SHAPE
    assert f(4, 4, FAKE, FAKE, 3, FAKE, None, None, None, None, None, 0, None) == BAD_SHAPE  # n_sps < B
    assert f(1024, 9, FAKE, FAKE, 20000, FAKE, None, None, None, None, None, 0, None) == BAD_SHAPE  # > 8192 pairs
    assert f(4, -1, FAKE, FAKE, 10, FAKE, None, None, None, None, None, 0, None) == BAD_SHAPE
    assert f(8193, 0, FAKE, FAKE, 9000, FAKE, None, None, None, None, None, 0, None) == BAD_SHAPE  # > 8192 requests
    need = L.dspark_prefix_schedule_workspace_size(4, 4)
    ws = FAKE if need else None
    assert f(4, 4, None, FAKE, 10, FAKE, None, None, None, None, ws, need, None) == NULL_ARG
    assert f(4, 4, FAKE, None, 10, FAKE, None, None, None, None, ws, need, None) == NULL_ARG
    assert f(4, 4, FAKE, FAKE, 10, None, None, None, None, None, ws, need, None) == NULL_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import draft_head_sampling_amd as dh

    monkeypatch.setattr(dh, "_lib", None)
    monkeypatch.setattr(dh, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dh.lib()


def _vf(L, B=2, gamma=3, V=100, dtype=1, d=FAKE, t=FAKE, x=FAKE, n=None, u=FAKE, G=FAKE, na=FAKE, nt=FAKE, ws=None,
        wsb=0):
    return L.dspark_verify(B, gamma, V, dtype, d, t, x, n, u, G, na, nt, None, ws, wsb, None)


def test_verify_host_checks(L):
    need = L.dspark_verify_workspace_size(2, 3, 100, 1)
    assert need > 0 and need % 256 == 0
    assert L.dspark_verify_workspace_size(65536, 3, 100, 1) == 0
    assert _vf(L, dtype=7) == BAD_DTYPE
    assert _vf(L, B=65536) == BAD_SHAPE
    assert _vf(L, gamma=4097) == BAD_SHAPE
    assert _vf(L, V=0) == BAD_SHAPE
    assert _vf(L, B=0) == OK  # nothing to do: nothing enqueued
    assert _vf(L) == WORKSPACE  # no workspace
    assert _vf(L, ws=FAKE * 256, wsb=need - 1) == WORKSPACE
    for kw in ("t", "G", "na", "nt", "d", "x", "u"):
        assert _vf(L, ws=FAKE * 256, wsb=need, **{kw: None}) == NULL_ARG, kw
    # gamma = 0: only the target row of the bonus draw is needed
    assert _vf(L, gamma=0, d=None, x=None, u=None, t=None, ws=FAKE * 256,
               wsb=L.dspark_verify_workspace_size(2, 0, 100, 1)) == NULL_ARG


def test_head_sample_gated_host_checks(L):
    need = L.dspark_head_sample_gated_workspace_size(4, 7, 100, 8, 16, 1)
    assert need > 0 and need % 256 == 0
    def g(**kw):
        a = dict(B=4, gamma=7, V=100, H=8, r=16, dtype=1, U=FAKE, h=FAKE, W1=FAKE, W2=FAKE, w=FAKE, Wg=FAKE, x0=FAKE,
                 tokens=FAKE, conf=FAKE, surv=FAKE, ws=None, wsb=0)
        a.update(kw)
        return L.dspark_head_sample_gated(a["B"], a["gamma"], a["V"], a["H"], a["r"], a["dtype"], a["U"], a["h"],
                                          a["W1"], a["W2"], a["w"], a["Wg"], 0.0, a["x0"], None, None, a["tokens"],
                                          a["conf"], a["surv"], None, None, a["ws"], a["wsb"], None)
    assert g(dtype=9) == BAD_DTYPE
    assert g(r=0) == BAD_SHAPE
    assert g(B=0) == OK
    assert g() == WORKSPACE
    assert g(ws=FAKE * 256, wsb=need, Wg=None) == NULL_ARG
    assert g(ws=FAKE * 256, wsb=need, h=None) == NULL_ARG


def test_head_sample_rnn_host_checks(L):
    need = L.dspark_head_sample_rnn_workspace_size(4, 7, 100, 8, 16, 1)
    assert need > L.dspark_head_sample_gated_workspace_size(4, 7, 100, 8, 16, 1) > 0 and need % 256 == 0
    def g(**kw):
        a = dict(B=4, gamma=7, V=100, H=8, r=16, dtype=1, Wrg=FAKE, Wrc=FAKE, ws=None, wsb=0)
        a.update(kw)
        return L.dspark_head_sample_rnn(a["B"], a["gamma"], a["V"], a["H"], a["r"], a["dtype"], FAKE, FAKE, FAKE,
                                        FAKE, FAKE, a["Wrg"], a["Wrc"], 0.0, FAKE, None, None, FAKE, FAKE, FAKE, None,
                                        None, a["ws"], a["wsb"], None)
    assert g(dtype=9) == BAD_DTYPE
    assert g(r=0) == BAD_SHAPE
    assert g(B=0) == OK
    assert g() == WORKSPACE
    assert g(ws=FAKE * 256, wsb=need, Wrg=None) == NULL_ARG
    assert g(ws=FAKE * 256, wsb=need, Wrc=None) == NULL_ARG


def _bl(L, N=2, gamma=3, V=100, H=8, r=256, dtype=1, U=FAKE, t=FAKE, h=FAKE, W1=FAKE, W2=FAKE, w=FAKE, xp=FAKE,
        y=FAKE, decay=4.0, ce=FAKE, l1=FAKE, conf=FAKE, bce=FAKE, loss=FAKE, ws=None, wsb=0):
    return L.dspark_block_loss(N, gamma, V, H, r, dtype, U, t, h, W1, W2, w, 0.0, xp, y, None, decay, 0.1, 0.9, 1.0,
                               ce, l1, conf, bce, loss, ws, wsb, None)


def test_block_loss_host_checks(L):
    need = L.dspark_block_loss_workspace_size(2, 3, 100, 8, 256, 1)
    assert need > 0 and need % 256 == 0
    assert L.dspark_block_loss_workspace_size(2, 3, 65535 * 512 + 1, 8, 256, 1) == 0
    assert _bl(L, dtype=0) == BAD_DTYPE  # bf16 only
    assert _bl(L, V=0) == BAD_SHAPE
    assert _bl(L, N=-1) == BAD_SHAPE
    assert _bl(L, decay=0.0) == BAD_SHAPE
    assert _bl(L, loss=None) == NULL_ARG
    for kw in ("U", "t", "h", "W1", "W2", "w", "xp", "y", "ce", "l1", "conf", "bce"):
        assert _bl(L, **{kw: None}) == NULL_ARG, kw
    assert _bl(L) == WORKSPACE
    assert _bl(L, ws=FAKE * 256, wsb=need - 1) == WORKSPACE
    assert _bl(L, r=128, ws=FAKE * 256, wsb=need) == BAD_SHAPE  # the tiles are rank 256
    assert _bl(L, W2=FAKE + 2, ws=FAKE * 256, wsb=need) == BAD_SHAPE  # 16-byte rows


def test_w2_bound_validation(L):
    """Host-side checks of dspark_w2_bound (nothing is enqueued)."""
    import ctypes
    buf = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks first
    assert L.dspark_w2_bound(1000, 256, 0, buf, buf, None) == 3  # fp32: bad dtype
    assert L.dspark_w2_bound(1000, 128, 1, buf, buf, None) == 2  # rank other than 256
    assert L.dspark_w2_bound(0, 256, 1, buf, buf, None) == 2     # empty vocabulary
    assert L.dspark_w2_bound(1000, 256, 1, None, buf, None) == 1
    assert L.dspark_w2_bound(1000, 256, 1, buf, None, None) == 1
    assert L.dspark_w2_bound(1000, 256, 1, ctypes.c_void_p(264), buf, None) == 2  # W2 not 16-byte aligned
