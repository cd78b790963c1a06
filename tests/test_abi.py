"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments synchronously with the documented status codes.

No call here reaches a kernel launch: every call is built to fail
validation, so these run on a host without a GPU.
"""
import os
import re

import pytest

import kv_cache_absorption_attn_amd as ispa
from kv_cache_absorption_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ispa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
A = 0x10000        # fake 16-byte aligned address, never dereferenced
MIS = 0x10008      # fake misaligned address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ispa_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ispa_attn_decomp", "ispa_gram_accumulate", "ispa_ridge_solve",
              "ispa_ridge_workspace_bytes", "ispa_layer_score", "ispa_apply_dW",
              "ispa_project", "ispa_status_string", "ispa_version"):
        assert n in names


def test_every_declared_symbol_is_exported():
    for n in declared_functions():
        assert hasattr(_lib.lib, n), n
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_status_strings():
    assert ispa.ispa_status_string(0) == "ok"
    for s in range(1, 8):
        assert ispa.ispa_status_string(s) not in ("ok", "unknown status")
    assert ispa.ispa_status_string(99) == "unknown status"
    assert ispa.ispa_version() >= 100


def attn(**kw):
    args = dict(q=A, n_q=16, ks=A, vs=A, n_sink=8, kc=A, vc=A, n_cur=8, kh=0, vh=0, n_hist=0,
                heads=2, d=128, scale=0.1, ol=A, ll=0, oh=0, lh=0, of=0, lf=0, do=0, stream=0)
    args.update(kw)
    return _lib.lib.ispa_attn_decomp(*args.values())


def test_attn_validation():
    assert attn(q=0) == NULL
    assert attn(d=96) == UNSUP
    assert attn(d=32) == UNSUP
    assert attn(n_sink=0, n_cur=0) == SHAPE
    assert attn(n_q=-1) == SHAPE
    assert attn(heads=0) == SHAPE
    assert attn(scale=0.0) == SHAPE
    assert attn(scale=float("nan")) == SHAPE
    assert attn(ol=0) == NULL                      # no output requested
    assert attn(n_hist=5) == NULL                  # history length without pointers
    assert attn(ks=0) == NULL
    assert attn(q=MIS) == ALIGN
    assert attn(ol=MIS) == ALIGN


def test_feature_major_validation():
    """The feature-major attention and Gram entry points: argument checks
    that return before any launch."""
    L = _lib.lib
    seg = (A, 16, A, A, 8, A, A, 8, 0, 0, 0, 2, 128, 0.1)

    def at(of=A, lf=0, xt=A, dt=A, ld=16):
        return L.ispa_attn_decomp_t(*seg, of, lf, xt, dt, ld, 0)
    assert at(xt=0) == NULL and at(dt=0) == NULL
    assert at(of=0) == NULL               # O_full is required
    assert at(ld=2 ** 22) == UNSUP        # 256 features x 2^22 tokens = 2 GiB
    assert at(ld=8) == SHAPE              # ld < n_q
    assert at(ld=20) == ALIGN             # ld % 8
    assert at(xt=MIS) == ALIGN
    assert L.ispa_attn_decomp_t(A, 16, A, A, 8, A, A, 8, 0, 0, 0, 2, 96, 0.1, A, 0, A, A, 16,
                                0) == UNSUP
    gt = L.ispa_gram_accumulate_t
    assert gt(0, A, 100, 104, 128, 1, A, A, 0, 1, 0) == NULL
    assert gt(A, A, 100, 96, 128, 1, A, A, 0, 1, 0) == SHAPE      # ld < n_tok
    assert gt(A, A, 100, 104, 120, 0, A, A, 0, 1, 0) == SHAPE     # no batch
    assert gt(A, A, 100, 104, 124, 1, A, A, 0, 1, 0) == UNSUP     # h % 8
    assert gt(A, A, 100, 102, 128, 1, A, A, 0, 1, 0) == ALIGN     # ld % 8
    assert gt(A, A, 100, 104, 128, 1, MIS, A, 0, 1, 0) == ALIGN
    assert gt(A, A, 100, 2 ** 20, 1024, 1, A, A, 0, 1, 0) == UNSUP  # 2 GiB per layer
    assert gt(A, A, 0, 104, 128, 1, A, A, 0, 0, 0) == OK          # nothing to add


def test_gram_validation():
    g = _lib.lib.ispa_gram_accumulate
    assert g(0, A, 10, 128, 1, A, A, 0, 0, 0) == NULL
    assert g(A, A, 10, 128, 1, 0, A, 0, 0, 0) == NULL
    assert g(A, A, 10, 0, 1, A, A, 0, 0, 0) == SHAPE
    assert g(A, A, -1, 128, 1, A, A, 0, 0, 0) == SHAPE
    assert g(A, A, 10, 128, 0, A, A, 0, 0, 0) == SHAPE
    assert g(A, A, 10, 100, 1, A, A, 0, 0, 0) == UNSUP
    assert g(A, MIS, 10, 128, 1, A, A, 0, 0, 0) == ALIGN
    assert g(A, A, 0, 128, 1, A, A, 0, 0, 0) == OK     # nothing to add, nothing launched


def test_ridge_validation():
    r = _lib.lib.ispa_ridge_solve
    need = ispa.ispa_ridge_workspace_bytes(2, 256)
    assert need > 3 * 2 * 256 * 256 * 4
    assert ispa.ispa_ridge_workspace_bytes(0, 256) == 0
    assert ispa.ispa_ridge_workspace_bytes(4, 256) > need
    assert r(2, 256, 0, A, A, 0.01, A, A, A, need, 0) == NULL
    assert r(0, 256, A, A, A, 0.01, A, A, A, need, 0) == SHAPE
    assert r(2, 256, A, A, A, -1.0, A, A, A, need, 0) == SHAPE
    assert r(2, 256, A, A, A, float("inf"), A, A, A, need, 0) == SHAPE
    assert r(2, 250, A, A, A, 0.01, A, A, A, need, 0) == UNSUP
    assert r(2, 256, A, A, A, 0.01, A, A, A, need - 1, 0) == WS
    assert r(2, 256, A, A, A, 0.01, A, A, 0, need, 0) == WS
    assert r(2, 256, A, A, MIS, 0.01, A, A, A, need, 0) == ALIGN


def test_score_apply_project_validation():
    s = _lib.lib.ispa_layer_score
    need = ispa.ispa_ridge_workspace_bytes(2, 256)
    assert s(2, 256, A, A, 0, A, A, 0.01, A, 1, A, need, A, A, A, 0) == NULL
    assert s(2, 256, A, A, A, A, A, 0.01, A, -1, A, need, A, A, A, 0) == SHAPE
    assert s(2, 256, A, A, A, A, A, 0.01, A, 1, A, 16, A, A, A, 0) == WS
    a = _lib.lib.ispa_apply_dW
    assert a(2, 256, 0, A, A, 0) == NULL
    assert a(0, 256, A, A, A, 0) == SHAPE
    assert a(2, 12, A, A, A, 0) == UNSUP
    p = _lib.lib.ispa_project
    assert p(A, A, 0, 4, 128, 128, 0) == NULL
    assert p(A, A, A, -4, 128, 128, 0) == SHAPE
    assert p(A, A, A, 4, 100, 128, 0) == UNSUP
    assert p(A, A, A, 0, 128, 128, 0) == OK


def test_fp8_attention_validation():
    """Argument checks of the E4M3 attention and the key mean that return
    before any launch."""
    wsb = ispa.ispa_attn_fp8_workspace_bytes
    need = wsb(100, 10, 20, 30, 2, 128)
    assert need >= 160 * 256 + 100 * 2 * 8
    assert wsb(100, 10, 20, 30, 2, 64) == 0 and wsb(-1, 0, 1, 0, 2, 128) == 0
    f = _lib.lib.ispa_attn_decomp_fp8
    base = [A, 100, A, A, 10, A, A, 20, A, A, 30, 2, 128, 0.1, 0, A, 0, 0, 0, A, 0, 0, A, need, 0]

    def call(**kw):
        names = ["q", "n_q", "ks", "vs", "n_sink", "kc", "vc", "n_cur", "kh", "vh", "n_hist",
                 "nh", "hd", "scale", "mean", "o_local", "lse_local", "o_hist", "lse_hist",
                 "o_full", "lse_full", "d_out", "ws", "ws_bytes", "stream"]
        args = list(base)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(hd=64) == UNSUP
    assert call(ws=0) == WS
    assert call(ws_bytes=need - 1) == WS
    assert call(mean=MIS) == ALIGN
    assert call(ws=MIS) == ALIGN
    assert call(q=0) == NULL
    assert call(o_local=0, o_full=0) == NULL
    assert call(scale=-1.0) == SHAPE
    assert call(n_sink=0, n_cur=0) == SHAPE
    assert call(n_q=0, ws=0, ws_bytes=0) == OK
    km = _lib.lib.ispa_key_mean
    kw = ispa.ispa_key_mean_workspace_bytes(2, 128)
    assert kw > 0 and ispa.ispa_key_mean_workspace_bytes(2, 64) == 0
    assert km(A, 10, A, 20, A, 30, 2, 128, 0, A, kw, 0) == NULL
    assert km(0, 10, A, 20, A, 30, 2, 128, A, A, kw, 0) == NULL
    assert km(A, 0, A, 0, A, 0, 2, 128, A, A, kw, 0) == SHAPE
    assert km(A, 10, 0, 0, 0, 0, 2, 64, A, A, kw, 0) == UNSUP
    assert km(A, 10, 0, 0, 0, 0, 2, 128, A, A, kw - 1, 0) == WS
    assert km(MIS, 10, 0, 0, 0, 0, 2, 128, A, A, kw, 0) == ALIGN


def test_grouped_validation():
    """Argument checks of the grouped launches that return before any launch."""
    L = _lib.lib
    job = _lib.AttnJob(q=A, n_q=10, k_sink=A, v_sink=A, n_sink=5, k_cur=A, v_cur=A, n_cur=5,
                       k_hist=0, v_hist=0, n_hist=0, o_full=A)
    jobs = (_lib.AttnJob * 9)(*([job] * 9))
    assert L.ispa_attn_decomp_grouped(None, 1, 2, 128, 0.1, 0) == NULL
    assert L.ispa_attn_decomp_grouped(jobs, 0, 2, 128, 0.1, 0) == SHAPE
    assert L.ispa_attn_decomp_grouped(jobs, 9, 2, 128, 0.1, 0) == SHAPE
    assert L.ispa_attn_decomp_grouped(jobs, 2, 2, 96, 0.1, 0) == UNSUP
    bad = (_lib.AttnJob * 2)(job, _lib.AttnJob(q=A, n_q=10, n_cur=5, k_cur=A, v_cur=A,
                                               o_full=MIS))
    assert L.ispa_attn_decomp_grouped(bad, 2, 2, 128, 0.1, 0) == ALIGN
    nothing = (_lib.AttnJob * 2)(_lib.AttnJob(q=A, n_q=10, n_cur=5, k_cur=A, v_cur=A),
                                 _lib.AttnJob(q=0, n_q=0, n_cur=5, k_cur=A, v_cur=A, o_full=A))
    assert L.ispa_attn_decomp_grouped(nothing, 2, 2, 128, 0.1, 0) == NULL   # job 0: no output
    empty = (_lib.AttnJob * 1)(_lib.AttnJob(q=0, n_q=0, n_cur=5, k_cur=A, v_cur=A, o_full=A))
    assert L.ispa_attn_decomp_grouped(empty, 1, 2, 128, 0.1, 0) == OK      # skipped
    pj = (_lib.ProjectJob * 9)(*([_lib.ProjectJob(x=A, w=A, y=A, n=4)] * 9))
    assert L.ispa_project_grouped(None, 1, 128, 128, 0) == NULL
    assert L.ispa_project_grouped(pj, 9, 128, 128, 0) == SHAPE
    assert L.ispa_project_grouped(pj, 2, 100, 128, 0) == UNSUP
    assert L.ispa_project_grouped(pj, 2, 128, 100, 0) == UNSUP
    assert L.ispa_project_grouped(pj, 2, 65536, 65536, 0) == UNSUP       # W above 2^31 bytes
    neg = (_lib.ProjectJob * 1)(_lib.ProjectJob(x=A, w=A, y=A, n=-1))
    assert L.ispa_project_grouped(neg, 1, 128, 128, 0) == SHAPE
    nul = (_lib.ProjectJob * 1)(_lib.ProjectJob(x=A, w=0, y=A, n=4))
    assert L.ispa_project_grouped(nul, 1, 128, 128, 0) == NULL
    mis = (_lib.ProjectJob * 1)(_lib.ProjectJob(x=A, w=A, y=MIS, n=4))
    assert L.ispa_project_grouped(mis, 1, 128, 128, 0) == ALIGN


def test_w8a8_validation():
    """Argument checks of the W8A8 calls that return before any launch."""
    qz = _lib.lib.ispa_quantize_fp8
    assert qz(A, 4, 64, 0, A, 0) == NULL
    assert qz(A, -1, 64, A, A, 0) == SHAPE
    assert qz(A, 4, 0, A, A, 0) == SHAPE
    assert qz(A, 4, 60, A, A, 0) == UNSUP
    assert qz(MIS, 4, 64, A, A, 0) == ALIGN
    assert qz(A, 0, 64, A, A, 0) == OK
    wsb = ispa.ispa_project_w8a8_workspace_bytes
    assert wsb(-1, 64) == 0 and wsb(10, 0) == 0
    need = wsb(100, 256)
    assert need >= 100 * 256 + 100 * 4
    pw = _lib.lib.ispa_project_w8a8
    assert pw(A, A, 0, A, 100, 256, 128, A, need, 0) == NULL
    assert pw(A, A, A, A, -1, 256, 128, A, need, 0) == SHAPE
    assert pw(A, A, A, A, 100, 96, 128, A, need, 0) == UNSUP
    assert pw(A, A, A, A, 100, 256, 100, A, need, 0) == UNSUP
    assert pw(A, A, A, A, 100, 256, 128, A, need - 1, 0) == WS
    assert pw(A, A, A, A, 100, 256, 128, 0, need, 0) == WS
    assert pw(A, A, A, MIS, 100, 256, 128, A, need, 0) == ALIGN
    assert pw(A, A, A, A, 0, 256, 128, 0, 0, 0) == OK
    # the allocation-free variant: the same checks, and sizes beyond its
    # fixed scratch, all before it looks up its scratch on a device
    na = _lib.lib.ispa_project_w8a8_noalloc
    assert na(A, A, 0, A, 100, 256, 128, 0) == NULL
    assert na(A, A, A, A, -1, 256, 128, 0) == SHAPE
    assert na(A, A, A, A, 100, 96, 128, 0) == UNSUP
    assert na(A, A, A, A, 100, 256, 100, 0) == UNSUP
    assert na(A, A, A, A, _lib.NOALLOC_MAX_TOKENS + 1, 64, 128, 0) == _lib.ISPA_ERR_SCRATCH
    rows = _lib.NOALLOC_MAX_CODE_BYTES // 5120 + 1
    assert na(A, A, A, A, rows, 5120, 128, 0) == _lib.ISPA_ERR_SCRATCH
    assert na(A, A, A, MIS, 100, 256, 128, 0) == ALIGN
    assert na(A, A, A, A, 0, 256, 128, 0) == OK


def test_kv_cache_validation():
    """Argument checks of the streaming KV cache that return before any HIP
    call: bad shapes, NULL handles and NULL outputs."""
    import ctypes as ct
    L = _lib.lib
    h = ct.c_void_p()
    assert L.ispa_kv_create(2, 2, 128, 8, 16, 32, None) == NULL
    assert L.ispa_kv_create(0, 2, 128, 8, 16, 32, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 0, 128, 8, 16, 32, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 2, 128, -1, 16, 32, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 2, 128, 8, 0, 32, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 2, 128, 8, 16, -16, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 2, 128, 8, 16, 40, ct.byref(h)) == SHAPE   # not whole chunks
    assert L.ispa_kv_create(2, 2, 128, 8, 1 << 40, 1 << 60, ct.byref(h)) == SHAPE
    assert L.ispa_kv_create(2, 2, 96, 8, 16, 32, ct.byref(h)) == UNSUP
    assert h.value is None
    view = _lib.KVView()
    assert L.ispa_kv_destroy(None) == NULL
    assert L.ispa_kv_view_of(None, 0, ct.byref(view)) == NULL
    assert L.ispa_kv_write(None, 0, 0, A, A, 0) == NULL
    assert L.ispa_kv_advance(None) == NULL
    assert L.ispa_kv_evict_history(None, 0, 0) == NULL
    assert L.ispa_kv_resident_bytes(None) == -1
    L.ispa_kv_last_error.restype = ct.c_char_p
    assert L.ispa_kv_last_error(None) == b""
    assert L.ispa_kv_attn(None, 0, A, 4, 0.1, A, 0, 0, 0, 0, 0, 0, 0) == NULL
    assert L.ispa_kv_layer_forward(None, 0, A, 4, 0.1, A, A, A, 0) == NULL
    assert ct.sizeof(_lib.KVView) == 4 * 8 + 6 * 8 + 3 * 8 + 8 + 2 * 4


def test_drift_and_session_validation():
    """Argument checks of the drift score and the streaming session that
    return before any HIP call."""
    import ctypes as ct
    L = _lib.lib
    assert ispa.ispa_drift_workspace_bytes(0, 128, 16) == 0
    need = ispa.ispa_drift_workspace_bytes(2, 128, 16)
    assert need >= ispa.ispa_ridge_workspace_bytes(2, 128)
    assert L.ispa_drift_prepare(2, 128, 0, 0.01, 10, A, A, A, A, need, 0) == NULL
    assert L.ispa_drift_prepare(2, 128, A, -1.0, 10, A, A, A, A, need, 0) == SHAPE
    assert L.ispa_drift_prepare(2, 128, A, 0.01, 0, A, A, A, A, need, 0) == SHAPE
    assert L.ispa_drift_prepare(2, 100, A, 0.01, 10, A, A, A, A, need, 0) == UNSUP
    assert L.ispa_drift_prepare(2, 128, A, 0.01, 10, A, A, A, A, 64, 0) == WS
    assert L.ispa_drift_prepare(2, 128, MIS, 0.01, 10, A, A, A, A, need, 0) == ALIGN
    rneed = ispa.ispa_ridge_workspace_bytes(2, 128)
    pf = L.ispa_drift_prepare_factored
    assert pf(2, 128, 0.01, 10, 0, A, A, rneed, 0) == NULL
    assert pf(2, 128, 0.01, 10, A, A, 0, rneed, 0) == NULL
    assert pf(0, 128, 0.01, 10, A, A, A, rneed, 0) == SHAPE
    assert pf(2, 128, float("inf"), 10, A, A, A, rneed, 0) == SHAPE
    assert pf(2, 128, 0.01, 0, A, A, A, rneed, 0) == SHAPE
    assert pf(2, 100, 0.01, 10, A, A, A, rneed, 0) == UNSUP
    assert pf(2, 128, 0.01, 10, A, A, A, rneed - 1, 0) == WS
    assert pf(2, 128, 0.01, 10, A, MIS, A, rneed, 0) == ALIGN
    assert L.ispa_drift_score(2, 128, A, A, 0, 16, 1, A, A, need, 0) == NULL
    assert L.ispa_drift_score(2, 128, A, A, A, 0, 1, A, A, need, 0) == SHAPE
    assert L.ispa_drift_score(2, 128, A, A, A, 16, 0, A, A, need, 0) == SHAPE
    assert L.ispa_drift_score(2, 128, A, A, A, 4096, 1, A, A, need, 0) == WS  # 4096 samples
    assert L.ispa_drift_score(2, 128, A, A, A, 16, 1, A, MIS, need, 0) == ALIGN
    assert L.ispa_drift_score(2, 128, A, A + 4, A, 16, 1, A, A, need, 0) == ALIGN  # ref: 8 B
    assert L.ispa_kv_restore_history(None, 0) == NULL

    cfg = _lib.SessionConfig(2, 2, 64, 1, 2, 0, 8, 16, 64, 0.125, 0.01, 4.0, 4)
    n = L.ispa_session_workspace_bytes(ct.byref(cfg))
    assert n > 0
    bad = _lib.SessionConfig(2, 2, 64, 3, 2, 0, 8, 16, 64, 0.125, 0.01, 4.0, 4)  # K > layers
    assert L.ispa_session_workspace_bytes(ct.byref(bad)) == 0
    h = ct.c_void_p()
    assert L.ispa_session_create(ct.byref(cfg), A, A, A, n, 0, None) == NULL
    assert L.ispa_session_create(ct.byref(cfg), 0, A, A, n, 0, ct.byref(h)) == NULL
    assert L.ispa_session_create(ct.byref(bad), A, A, A, n, 0, ct.byref(h)) == SHAPE
    d96 = _lib.SessionConfig(2, 2, 96, 1, 2, 0, 8, 16, 64, 0.125, 0.01, 4.0, 4)
    assert L.ispa_session_create(ct.byref(d96), A, A, A, n, 0, ct.byref(h)) == UNSUP
    assert L.ispa_session_create(ct.byref(cfg), A, A, A, n - 1, 0, ct.byref(h)) == WS
    assert L.ispa_session_create(ct.byref(cfg), MIS, A, A, n, 0, ct.byref(h)) == ALIGN
    # quantized variant: unknown flag bits, head_dim 64 with E4M3 attention,
    # and the workspace that the flags add
    unk = _lib.SessionConfig(2, 2, 64, 1, 2, 4, 8, 16, 64, 0.125, 0.01, 4.0, 4)
    assert L.ispa_session_workspace_bytes(ct.byref(unk)) == 0
    assert L.ispa_session_create(ct.byref(unk), A, A, A, n, 0, ct.byref(h)) == SHAPE
    f8 = _lib.SessionConfig(2, 2, 64, 1, 2, _lib.SESSION_FP8_ATTN, 8, 16, 64, 0.125, 0.01, 4.0, 4)
    n8 = L.ispa_session_workspace_bytes(ct.byref(f8))
    assert n8 > n
    assert L.ispa_session_create(ct.byref(f8), A, A, A, n8, 0, ct.byref(h)) == UNSUP
    q = _lib.SessionConfig(2, 1, 128, 1, 2, _lib.SESSION_W8A8 | _lib.SESSION_FP8_ATTN, 8, 16, 64,
                           0.125, 0.01, 4.0, 4)
    nq = L.ispa_session_workspace_bytes(ct.byref(q))
    assert nq >= n + 2 * 128 * 128
    assert L.ispa_session_create(ct.byref(q), A, A, A, nq - 1, 0, ct.byref(h)) == WS
    assert h.value is None
    st = _lib.SessionState()
    assert L.ispa_session_destroy(None) == NULL
    assert L.ispa_session_cache(None) is None
    assert L.ispa_session_layer(None, 0, A, A, 0) == NULL
    assert L.ispa_session_end_chunk(None, 0, None) == NULL
    assert L.ispa_session_query(None, ct.byref(st), None, None, None) == NULL
    g = L.ispa_session_layer_grouped
    ptrs = (ct.c_void_p * 9)(*([A] * 9))
    nulls = (ct.c_void_p * 2)(None, None)
    assert g(None, 1, 0, ptrs, ptrs, 0) == NULL
    assert g(ptrs, 1, 0, None, ptrs, 0) == NULL
    assert g(ptrs, 0, 0, ptrs, ptrs, 0) == SHAPE
    assert g(ptrs, 9, 0, ptrs, ptrs, 0) == SHAPE
    assert g(nulls, 2, 0, ptrs, ptrs, 0) == NULL     # a NULL session, never dereferenced
    assert ct.sizeof(_lib.SessionConfig) == 6 * 4 + 3 * 8 + 2 * 4 + 8 + 8
    assert ct.sizeof(_lib.SessionState) == 4 * 4 + 8
