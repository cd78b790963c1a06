"""ctypes binding of libispa.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
dtype / shape / contiguity, and forwards raw device pointers plus the current
HIP stream to the C entry point of the same name (declared in
include/ispa.h). All arithmetic runs in the library's HIP kernels; there is
no fallback path. A missing or unloadable library raises ImportError.
"""
from __future__ import annotations

import ctypes as ct
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libispa.so")

ISPA_OK = 0
ISPA_ERR_NULL = 1
ISPA_ERR_SHAPE = 2
ISPA_ERR_UNSUPPORTED = 3
ISPA_ERR_ALIGN = 4
ISPA_ERR_WORKSPACE = 5
ISPA_ERR_HIP = 6
ISPA_ERR_SCRATCH = 7
NOALLOC_MAX_CODE_BYTES = 32 * 1024 * 1024
NOALLOC_MAX_TOKENS = 65536

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python kv_cache_absorption_attn_amd/build.py`")
try:
    lib = ct.CDLL(LIB_PATH)
except OSError as exc:  # pragma: no cover - depends on the ROCm install
    raise ImportError(f"cannot load {LIB_PATH}: {exc}") from exc

_p, _i, _i64, _f, _sz = ct.c_void_p, ct.c_int, ct.c_int64, ct.c_float, ct.c_size_t

lib.ispa_status_string.restype = ct.c_char_p
lib.ispa_status_string.argtypes = [_i]
lib.ispa_version.restype = _i
lib.ispa_version.argtypes = []
lib.ispa_attn_decomp.restype = _i
lib.ispa_attn_decomp.argtypes = [_p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _p, _i64, _i, _i, _f,
                                 _p, _p, _p, _p, _p, _p, _p, _p]
lib.ispa_attn_fp8_workspace_bytes.restype = _sz
lib.ispa_attn_fp8_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i, _i]
lib.ispa_attn_decomp_fp8.restype = _i
lib.ispa_attn_decomp_fp8.argtypes = [_p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _p, _i64, _i, _i,
                                     _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
lib.ispa_key_mean_workspace_bytes.restype = _sz
lib.ispa_key_mean_workspace_bytes.argtypes = [_i, _i]
lib.ispa_key_mean.restype = _i
lib.ispa_key_mean.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i, _i, _p, _p, _sz, _p]


class AttnJob(ct.Structure):
    """ispa_attn_job: one call of a grouped attention launch."""
    _fields_ = [("q", ct.c_void_p), ("n_q", ct.c_int64),
                ("k_sink", ct.c_void_p), ("v_sink", ct.c_void_p),
                ("n_sink", ct.c_int64),
                ("k_cur", ct.c_void_p), ("v_cur", ct.c_void_p), ("n_cur", ct.c_int64),
                ("k_hist", ct.c_void_p), ("v_hist", ct.c_void_p),
                ("n_hist", ct.c_int64),
                ("o_local", ct.c_void_p), ("lse_local", ct.c_void_p),
                ("o_hist", ct.c_void_p), ("lse_hist", ct.c_void_p),
                ("o_full", ct.c_void_p), ("lse_full", ct.c_void_p),
                ("d_out", ct.c_void_p)]


class ProjectJob(ct.Structure):
    """ispa_project_job: one product of a grouped projection launch."""
    _fields_ = [("x", ct.c_void_p), ("w", ct.c_void_p), ("y", ct.c_void_p),
                ("n", ct.c_int64)]


MAX_GROUP = 8
lib.ispa_attn_decomp_grouped.restype = _i
lib.ispa_attn_decomp_grouped.argtypes = [ct.POINTER(AttnJob), _i, _i, _i, _f, _p]
lib.ispa_project_grouped.restype = _i
lib.ispa_project_grouped.argtypes = [ct.POINTER(ProjectJob), _i, _i, _i, _p]
lib.ispa_session_layer_grouped.restype = _i
lib.ispa_session_layer_grouped.argtypes = [_p, _i, _i, _p, _p, _p]
lib.ispa_gram_accumulate.restype = _i
lib.ispa_gram_accumulate.argtypes = [_p, _p, _i64, _i, _i, _p, _p, _p, _i, _p]
lib.ispa_gram_accumulate_t.restype = _i
lib.ispa_gram_accumulate_t.argtypes = [_p, _p, _i64, _i64, _i, _i, _p, _p, _p, _i, _p]
lib.ispa_attn_decomp_t.restype = _i
lib.ispa_attn_decomp_t.argtypes = [_p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _p, _i64, _i, _i, _f,
                                   _p, _p, _p, _p, _i64, _p]
lib.ispa_ridge_workspace_bytes.restype = _sz
lib.ispa_ridge_workspace_bytes.argtypes = [_i, _i]
lib.ispa_ridge_solve.restype = _i
lib.ispa_ridge_solve.argtypes = [_i, _i, _p, _p, _p, _f, _p, _p, _p, _sz, _p]
lib.ispa_layer_score.restype = _i
lib.ispa_layer_score.argtypes = [_i, _i, _p, _p, _p, _p, _p, _f, _p, _i, _p, _sz, _p, _p, _p, _p]
lib.ispa_apply_dW.restype = _i
lib.ispa_apply_dW.argtypes = [_i, _i, _p, _p, _p, _p]
lib.ispa_project.restype = _i
lib.ispa_project.argtypes = [_p, _p, _p, _i64, _i, _i, _p]



class KVView(ct.Structure):
    """Mirror of ispa_kv_view (include/ispa.h)."""
    _fields_ = [("k_sink", _p), ("v_sink", _p), ("k_cur", _p), ("v_cur", _p),
                ("seg_k", _p * 3), ("seg_v", _p * 3), ("seg_n", _i64 * 3),
                ("n_hist", _i64), ("split_ok", ct.c_int32), ("local_only", ct.c_int32)]


lib.ispa_kv_create.restype = _i
lib.ispa_kv_create.argtypes = [_i, _i, _i, _i64, _i64, _i64, ct.POINTER(_p)]
lib.ispa_kv_destroy.restype = _i
lib.ispa_kv_destroy.argtypes = [_p]
lib.ispa_kv_view_of.restype = _i
lib.ispa_kv_view_of.argtypes = [_p, _i, ct.POINTER(KVView)]
lib.ispa_kv_write.restype = _i
lib.ispa_kv_write.argtypes = [_p, _i, _i, _p, _p, _p]
lib.ispa_kv_advance.restype = _i
lib.ispa_kv_advance.argtypes = [_p]
lib.ispa_kv_evict_history.restype = _i
lib.ispa_kv_evict_history.argtypes = [_p, _i, _p]
lib.ispa_quantize_fp8.restype = _i
lib.ispa_quantize_fp8.argtypes = [_p, _i64, _i, _p, _p, _p]
lib.ispa_project_w8a8_workspace_bytes.restype = _sz
lib.ispa_project_w8a8_workspace_bytes.argtypes = [_i64, _i]
lib.ispa_project_w8a8.restype = _i
lib.ispa_project_w8a8.argtypes = [_p, _p, _p, _p, _i64, _i, _i, _p, _sz, _p]
lib.ispa_project_w8a8_noalloc.restype = _i
lib.ispa_project_w8a8_noalloc.argtypes = [_p, _p, _p, _p, _i64, _i, _i, _p]
lib.ispa_kv_restore_history.restype = _i
lib.ispa_kv_restore_history.argtypes = [_p, _i]
lib.ispa_drift_workspace_bytes.restype = _sz
lib.ispa_drift_workspace_bytes.argtypes = [_i, _i, _i64]
lib.ispa_drift_prepare.restype = _i
lib.ispa_drift_prepare.argtypes = [_i, _i, _p, _f, _i64, _p, _p, _p, _p, _sz, _p]
lib.ispa_drift_prepare_factored.restype = _i
lib.ispa_drift_prepare_factored.argtypes = [_i, _i, _f, _i64, _p, _p, _p, _sz, _p]
lib.ispa_drift_score.restype = _i
lib.ispa_drift_score.argtypes = [_i, _i, _p, _p, _p, _i64, _i64, _p, _p, _sz, _p]


class SessionConfig(ct.Structure):
    """Mirror of ispa_session_config (include/ispa.h)."""
    _fields_ = [("n_layers", ct.c_int32), ("n_heads", ct.c_int32), ("head_dim", ct.c_int32),
                ("k_select", ct.c_int32), ("t_warm", ct.c_int32), ("flags", ct.c_int32),
                ("n_sink", _i64), ("n_cur", _i64), ("hist_capacity", _i64),
                ("sm_scale", ct.c_float), ("lam", ct.c_float), ("drift_threshold", ct.c_double),
                ("drift_stride", _i64)]


SESSION_W8A8 = 1        # ISPA_SESSION_W8A8: E4M3 projections
SESSION_FP8_ATTN = 2    # ISPA_SESSION_FP8_ATTN: E4M3 attention while streaming


class SessionState(ct.Structure):
    """Mirror of ispa_session_state (include/ispa.h)."""
    _fields_ = [("phase", ct.c_int32), ("warm_count", ct.c_int32),
                ("n_calibrations", ct.c_int32), ("reserved", ct.c_int32), ("chunk", _i64)]


lib.ispa_session_workspace_bytes.restype = _sz
lib.ispa_session_workspace_bytes.argtypes = [ct.POINTER(SessionConfig)]
lib.ispa_session_create.restype = _i
lib.ispa_session_create.argtypes = [ct.POINTER(SessionConfig), _p, _p, _p, _sz, _p,
                                    ct.POINTER(_p)]
lib.ispa_session_destroy.restype = _i
lib.ispa_session_destroy.argtypes = [_p]
lib.ispa_session_cache.restype = _p
lib.ispa_session_cache.argtypes = [_p]
lib.ispa_session_layer.restype = _i
lib.ispa_session_layer.argtypes = [_p, _i, _p, _p, _p]
lib.ispa_session_end_chunk.restype = _i
lib.ispa_session_end_chunk.argtypes = [_p, _p, ct.POINTER(_i)]
lib.ispa_session_query.restype = _i
lib.ispa_session_query.argtypes = [_p, ct.POINTER(SessionState), _p, _p, _p]

ISPA_PHASE_WARMUP, ISPA_PHASE_STREAM = 0, 1
ISPA_EVENT_NONE, ISPA_EVENT_ABSORBED, ISPA_EVENT_RECALIBRATE = 0, 1, 2

lib.ispa_kv_last_error.restype = ct.c_char_p
lib.ispa_kv_last_error.argtypes = [_p]
lib.ispa_kv_resident_bytes.restype = _i64
lib.ispa_kv_resident_bytes.argtypes = [_p]
lib.ispa_kv_attn.restype = _i
lib.ispa_kv_attn.argtypes = [_p, _i, _p, _i64, _f, _p, _p, _p, _p, _p, _p, _p, _p]
lib.ispa_kv_layer_forward.restype = _i
lib.ispa_kv_layer_forward.argtypes = [_p, _i, _p, _i64, _f, _p, _p, _p, _p]

ISPA_KV_CURRENT = 0
ISPA_KV_SINK = 1

EXPORTED = ("ispa_status_string", "ispa_version", "ispa_attn_decomp", "ispa_gram_accumulate",
            "ispa_ridge_workspace_bytes", "ispa_ridge_solve", "ispa_layer_score",
            "ispa_apply_dW", "ispa_project", "ispa_kv_create", "ispa_kv_destroy",
            "ispa_kv_view_of", "ispa_kv_write", "ispa_kv_advance", "ispa_kv_evict_history",
            "ispa_kv_last_error", "ispa_kv_resident_bytes", "ispa_kv_attn",
            "ispa_kv_layer_forward", "ispa_kv_restore_history", "ispa_drift_workspace_bytes",
            "ispa_drift_prepare", "ispa_drift_prepare_factored", "ispa_drift_score", "ispa_session_workspace_bytes",
            "ispa_session_create", "ispa_session_destroy", "ispa_session_cache",
            "ispa_session_layer", "ispa_session_end_chunk", "ispa_session_query",
            "ispa_quantize_fp8", "ispa_project_w8a8_workspace_bytes", "ispa_project_w8a8",
            "ispa_attn_fp8_workspace_bytes", "ispa_attn_decomp_fp8",
            "ispa_key_mean_workspace_bytes", "ispa_key_mean", "ispa_attn_decomp_grouped",
            "ispa_project_grouped", "ispa_session_layer_grouped", "ispa_project_w8a8_noalloc",
            "ispa_attn_decomp_t", "ispa_gram_accumulate_t")


class IspaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        msg = f"{fn}: {ispa_status_string(status)} (status {status})"
        super().__init__(msg + (f" [{detail}]" if detail else ""))
        self.status = status


def ispa_status_string(status: int) -> str:
    return lib.ispa_status_string(int(status)).decode()


def ispa_version() -> int:
    return int(lib.ispa_version())


def _check(fn: str, status: int) -> None:
    if status != ISPA_OK:
        raise IspaError(fn, status)


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _attn_args(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist, outs):
    bf = torch.bfloat16
    o_local, lse_local, o_hist, lse_hist, o_full, lse_full, d_out = outs
    n_q, n_heads, head_dim = q.shape
    segs = []
    for name, k, v in (("sink", k_sink, v_sink), ("cur", k_cur, v_cur), ("hist", k_hist, v_hist)):
        n = 0 if k is None else k.shape[0]
        if k is not None and (k.shape[1:] != q.shape[1:] or v.shape != k.shape):
            raise ValueError(f"k_{name}/v_{name} shape mismatch")
        segs += [_ptr(k, bf, "k_" + name) if n else 0, _ptr(v, bf, "v_" + name) if n else 0, n]
    for name, t, dt in (("o_local", o_local, bf), ("o_hist", o_hist, bf), ("o_full", o_full, bf),
                        ("d_out", d_out, bf)):
        if t is not None and tuple(t.shape) != (n_q, n_heads * head_dim):
            raise ValueError(f"{name}: expected shape {(n_q, n_heads * head_dim)}")
    for name, t in (("lse_local", lse_local), ("lse_hist", lse_hist), ("lse_full", lse_full)):
        if t is not None and tuple(t.shape) != (n_heads, n_q):
            raise ValueError(f"{name}: expected shape {(n_heads, n_q)}")
    f32 = torch.float32
    out_ptrs = [_ptr(o_local, bf, "o_local"), _ptr(lse_local, f32, "lse_local"),
                _ptr(o_hist, bf, "o_hist"), _ptr(lse_hist, f32, "lse_hist"),
                _ptr(o_full, bf, "o_full"), _ptr(lse_full, f32, "lse_full"),
                _ptr(d_out, bf, "d_out")]
    return n_q, n_heads, head_dim, segs, out_ptrs


def ispa_attn_decomp(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist, sm_scale: float, *,
                     o_local=None, lse_local=None, o_hist=None, lse_hist=None, o_full=None,
                     lse_full=None, d_out=None, stream=None) -> None:
    """q [n_q, H, d]; k_*/v_* [n, H, d] bf16 (k_hist/v_hist may have n = 0).
    Outputs are preallocated tensors: o_* / d_out [n_q, H*d] bf16, lse_*
    [H, n_q] fp32; pass the ones to produce."""
    n_q, n_heads, head_dim, segs, outs = _attn_args(
        q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist,
        (o_local, lse_local, o_hist, lse_hist, o_full, lse_full, d_out))
    st = lib.ispa_attn_decomp(_ptr(q, torch.bfloat16, "q"), n_q, *segs, n_heads, head_dim,
                              float(sm_scale), *outs, _stream(stream))
    _check("ispa_attn_decomp", st)


def ispa_attn_decomp_t(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist, sm_scale: float, xt,
                       dt, *, o_full, col: int = 0, lse_full=None, stream=None) -> None:
    """The warmup step's attention with X = O_local and D written
    feature-major: xt, dt are [H*d, ld] bf16 tensors and this call fills
    their columns [col, col + n_q) (col % 8 == 0), so the warmup steps of one
    layer can sit side by side; o_full [n_q, H*d] bf16 is required (the
    kernel keeps X in it until the merge), lse_full optional as in
    ispa_attn_decomp."""
    n_q, n_heads, head_dim, segs, outs = _attn_args(
        q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist,
        (None, None, None, None, o_full, lse_full, None))
    h = n_heads * head_dim
    for name, t in (("xt", xt), ("dt", dt)):
        if t.dim() != 2 or t.shape[0] != h or t.shape[1] < col + n_q:
            raise ValueError(f"{name}: expected [{h}, >= {col + n_q}]")
    if dt.shape != xt.shape or col < 0:
        raise ValueError("ispa_attn_decomp_t: xt / dt / col mismatch")
    ld = xt.shape[1]
    st = lib.ispa_attn_decomp_t(_ptr(q, torch.bfloat16, "q"), n_q, *segs, n_heads, head_dim,
                                float(sm_scale), outs[4], outs[5],
                                _ptr(xt, torch.bfloat16, "xt") + 2 * col,
                                _ptr(dt, torch.bfloat16, "dt") + 2 * col, ld, _stream(stream))
    _check("ispa_attn_decomp_t", st)


def ispa_attn_decomp_grouped(calls, sm_scale: float, *, stream=None) -> None:
    """Several attention calls in one launch. `calls` is a list of dicts with
    the arguments of ispa_attn_decomp: q, k_sink, v_sink, k_cur, v_cur,
    k_hist, v_hist and any of the outputs (same heads and head_dim)."""
    if not 1 <= len(calls) <= MAX_GROUP:
        raise ValueError(f"ispa_attn_decomp_grouped: 1..{MAX_GROUP} calls")
    jobs = (AttnJob * len(calls))()
    shape = None
    for j, c in zip(jobs, calls):
        q = c["q"]
        if shape is not None and q.shape[1:] != shape:
            raise ValueError("ispa_attn_decomp_grouped: heads / head_dim differ between calls")
        shape = q.shape[1:]
        n_q, _, _, segs, outs = _attn_args(
            q, c.get("k_sink"), c.get("v_sink"), c.get("k_cur"), c.get("v_cur"),
            c.get("k_hist"), c.get("v_hist"),
            tuple(c.get(k) for k in ("o_local", "lse_local", "o_hist", "lse_hist", "o_full",
                                     "lse_full", "d_out")))
        j.q, j.n_q = _ptr(q, torch.bfloat16, "q"), n_q
        j.k_sink, j.v_sink, j.n_sink, j.k_cur, j.v_cur, j.n_cur, j.k_hist, j.v_hist, \
            j.n_hist = segs
        j.o_local, j.lse_local, j.o_hist, j.lse_hist, j.o_full, j.lse_full, j.d_out = outs
    st = lib.ispa_attn_decomp_grouped(jobs, len(calls), shape[0], shape[1], float(sm_scale),
                                      _stream(stream))
    _check("ispa_attn_decomp_grouped", st)


def ispa_project_grouped(xs, ws, ys, *, stream=None) -> None:
    """ys[g] [n_g, h_out] = xs[g] [n_g, h_in] ws[g]^T for every g, one launch."""
    if not 1 <= len(xs) <= MAX_GROUP or not len(xs) == len(ws) == len(ys):
        raise ValueError(f"ispa_project_grouped: 1..{MAX_GROUP} products")
    h_out, h_in = ws[0].shape
    jobs = (ProjectJob * len(xs))()
    for j, x, w, y in zip(jobs, xs, ws, ys):
        if tuple(w.shape) != (h_out, h_in) or x.shape[1] != h_in or \
                tuple(y.shape) != (x.shape[0], h_out):
            raise ValueError("ispa_project_grouped: shape mismatch")
        j.x, j.w, j.y = (_ptr(x, torch.bfloat16, "x"), _ptr(w, torch.bfloat16, "w"),
                         _ptr(y, torch.bfloat16, "y"))
        j.n = x.shape[0]
    st = lib.ispa_project_grouped(jobs, len(xs), h_in, h_out, _stream(stream))
    _check("ispa_project_grouped", st)


def ispa_attn_fp8_workspace_bytes(n_q: int, n_sink: int, n_cur: int, n_hist: int,
                                  n_heads: int, head_dim: int) -> int:
    return int(lib.ispa_attn_fp8_workspace_bytes(n_q, n_sink, n_cur, n_hist, n_heads, head_dim))


def ispa_attn_decomp_fp8(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist, sm_scale: float,
                         workspace, *, k_mean=None, o_local=None, lse_local=None, o_hist=None,
                         lse_hist=None, o_full=None, lse_full=None, d_out=None,
                         stream=None) -> None:
    """ispa_attn_decomp with E4M3 scores; k_mean [H, d] bf16 (or None) is the
    smoothing vector, workspace a uint8 tensor of
    ispa_attn_fp8_workspace_bytes(...) bytes."""
    n_q, n_heads, head_dim, segs, outs = _attn_args(
        q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist,
        (o_local, lse_local, o_hist, lse_hist, o_full, lse_full, d_out))
    if k_mean is not None and tuple(k_mean.shape) != (n_heads, head_dim):
        raise ValueError("k_mean: expected shape (n_heads, head_dim)")
    st = lib.ispa_attn_decomp_fp8(
        _ptr(q, torch.bfloat16, "q"), n_q, *segs, n_heads, head_dim, float(sm_scale),
        _ptr(k_mean, torch.bfloat16, "k_mean"), *outs, _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_attn_decomp_fp8", st)


def ispa_key_mean_workspace_bytes(n_heads: int, head_dim: int) -> int:
    return int(lib.ispa_key_mean_workspace_bytes(n_heads, head_dim))


def ispa_key_mean(k_sink, k_cur, k_hist, mu, workspace, *, stream=None) -> None:
    """mu [H, d] bf16 = mean of the keys of the given segments ([n, H, d] bf16,
    any may be None)."""
    segs = []
    shape = None
    for name, k in (("k_sink", k_sink), ("k_cur", k_cur), ("k_hist", k_hist)):
        n = 0 if k is None else k.shape[0]
        if k is not None:
            if shape is not None and k.shape[1:] != shape:
                raise ValueError("ispa_key_mean: segment shapes differ")
            shape = k.shape[1:]
        segs += [_ptr(k, torch.bfloat16, name) if n else 0, n]
    if shape is None:
        raise ValueError("ispa_key_mean: no keys")
    n_heads, head_dim = shape
    if tuple(mu.shape) != (n_heads, head_dim):
        raise ValueError("mu: expected shape (n_heads, head_dim)")
    st = lib.ispa_key_mean(*segs, n_heads, head_dim, _ptr(mu, torch.bfloat16, "mu"),
                           _ptr(workspace, None, "workspace"),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_key_mean", st)


def ispa_gram_accumulate(x, d, G, C, E=None, *, zero_first: bool = False, stream=None) -> None:
    """x, d [B, n_tok, h] (or [n_tok, h]) bf16; G, C, E [B, h, h] fp32."""
    if x.dim() == 2:
        x, d = x.unsqueeze(0), d.unsqueeze(0)
        G, C = G.unsqueeze(0), C.unsqueeze(0)
        E = None if E is None else E.unsqueeze(0)
    b, n_tok, h = x.shape
    if d.shape != x.shape or G.shape != (b, h, h) or C.shape != (b, h, h) or (
            E is not None and E.shape != (b, h, h)):
        raise ValueError("ispa_gram_accumulate: shape mismatch")
    st = lib.ispa_gram_accumulate(_ptr(x, torch.bfloat16, "x"), _ptr(d, torch.bfloat16, "d"),
                                  n_tok, h, b, _ptr(G, torch.float32, "G"),
                                  _ptr(C, torch.float32, "C"), _ptr(E, torch.float32, "E"),
                                  1 if zero_first else 0, _stream(stream))
    _check("ispa_gram_accumulate", st)


def ispa_gram_accumulate_t(xt, dt, n_tok: int, G, C, E=None, *, zero_first: bool = False,
                           stream=None) -> None:
    """xt, dt [B, h, ld] (or [h, ld]) bf16 feature-major activations, the
    first n_tok columns used; G, C, E [B, h, h] fp32."""
    if xt.dim() == 2:
        xt, dt = xt.unsqueeze(0), dt.unsqueeze(0)
        G, C = G.unsqueeze(0), C.unsqueeze(0)
        E = None if E is None else E.unsqueeze(0)
    b, h, ld = xt.shape
    if dt.shape != xt.shape or G.shape != (b, h, h) or C.shape != (b, h, h) or (
            E is not None and E.shape != (b, h, h)):
        raise ValueError("ispa_gram_accumulate_t: shape mismatch")
    st = lib.ispa_gram_accumulate_t(_ptr(xt, torch.bfloat16, "xt"), _ptr(dt, torch.bfloat16, "dt"),
                                    n_tok, ld, h, b, _ptr(G, torch.float32, "G"),
                                    _ptr(C, torch.float32, "C"), _ptr(E, torch.float32, "E"),
                                    1 if zero_first else 0, _stream(stream))
    _check("ispa_gram_accumulate_t", st)


def ispa_ridge_workspace_bytes(n_layers: int, h: int) -> int:
    return int(lib.ispa_ridge_workspace_bytes(n_layers, h))


def ispa_ridge_solve(G, C, Wo, lam: float, dW, info, workspace, *, stream=None) -> None:
    """G, C [L, h, h] fp32; Wo [L, h, h] bf16; dW [L, h, h] fp32 out;
    info [L] int32 out; workspace uint8 tensor of ispa_ridge_workspace_bytes."""
    n_layers, h, _ = G.shape
    st = lib.ispa_ridge_solve(n_layers, h, _ptr(G, torch.float32, "G"),
                              _ptr(C, torch.float32, "C"), _ptr(Wo, torch.bfloat16, "Wo"),
                              float(lam), _ptr(dW, torch.float32, "dW"),
                              _ptr(info, torch.int32, "info"), _ptr(workspace, None, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_ridge_solve", st)


def ispa_layer_score(G, C, E, Wo, dW, lam: float, info, K: int, workspace, eps_abs, eps_rel,
                     selected, *, stream=None) -> None:
    n_layers, h, _ = G.shape
    st = lib.ispa_layer_score(n_layers, h, _ptr(G, torch.float32, "G"),
                              _ptr(C, torch.float32, "C"), _ptr(E, torch.float32, "E"),
                              _ptr(Wo, torch.bfloat16, "Wo"), _ptr(dW, torch.float32, "dW"),
                              float(lam), _ptr(info, torch.int32, "info"), int(K),
                              _ptr(workspace, None, "workspace"),
                              workspace.numel() * workspace.element_size(),
                              _ptr(eps_abs, torch.float64, "eps_abs"),
                              _ptr(eps_rel, torch.float64, "eps_rel"),
                              _ptr(selected, torch.int32, "selected"), _stream(stream))
    _check("ispa_layer_score", st)


def ispa_apply_dW(selected, dW, Wo, *, stream=None) -> None:
    n_layers, h, _ = Wo.shape
    st = lib.ispa_apply_dW(n_layers, h, _ptr(selected, torch.int32, "selected"),
                           _ptr(dW, torch.float32, "dW"), _ptr(Wo, torch.bfloat16, "Wo"),
                           _stream(stream))
    _check("ispa_apply_dW", st)


def ispa_project(x, w, y, *, stream=None) -> None:
    """y [n, h_out] = x [n, h_in] @ w[h_out, h_in]^T, all bf16."""
    n, h_in = x.shape
    h_out = w.shape[0]
    if w.shape[1] != h_in or tuple(y.shape) != (n, h_out):
        raise ValueError("ispa_project: shape mismatch")
    st = lib.ispa_project(_ptr(x, torch.bfloat16, "x"), _ptr(w, torch.bfloat16, "w"),
                          _ptr(y, torch.bfloat16, "y"), n, h_in, h_out, _stream(stream))
    _check("ispa_project", st)


class KVCache:
    """Streaming KV cache of n_layers attention layers (ispa_kv_* in
    include/ispa.h): sink, current chunk and history rows of every layer,
    with the history's device memory mapped as it grows and released when a
    layer turns local-only. The handle is freed by close() (or when the
    object is collected)."""

    def __init__(self, n_layers: int, n_heads: int, head_dim: int, n_sink: int, n_cur: int,
                 hist_capacity: int):
        h = _p()
        self._h = _p()
        st = lib.ispa_kv_create(n_layers, n_heads, head_dim, n_sink, n_cur, hist_capacity,
                                ct.byref(h))
        if st != ISPA_OK:
            raise IspaError("ispa_kv_create", st, lib.ispa_kv_last_error(None).decode())
        self._h = h
        self.n_layers, self.n_heads, self.head_dim = n_layers, n_heads, head_dim
        self.n_sink, self.n_cur, self.hist_capacity = n_sink, n_cur, hist_capacity

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("KVCache is closed")
        return self._h.value

    def _check(self, fn: str, status: int) -> None:
        if status != ISPA_OK:
            raise IspaError(fn, status, lib.ispa_kv_last_error(self._h).decode())

    def close(self) -> None:
        if getattr(self, "_h", None):
            st = lib.ispa_kv_destroy(self._h)
            self._h = _p()
            _check("ispa_kv_destroy", st)

    def __del__(self):  # pragma: no cover - depends on collection order
        try:
            self.close()
        except Exception:
            pass

    def view(self, layer: int) -> KVView:
        v = KVView()
        _check("ispa_kv_view_of", lib.ispa_kv_view_of(self.handle, layer, ct.byref(v)))
        return v

    def _rows(self, t, n, name):
        if tuple(t.shape) != (n, self.n_heads, self.head_dim):
            raise ValueError(f"{name}: expected shape {(n, self.n_heads, self.head_dim)}")
        return _ptr(t, torch.bfloat16, name)

    def write(self, layer: int, k, v, *, sink: bool = False, stream=None) -> None:
        """Copy k, v [rows, n_heads, head_dim] bf16 into the layer's current
        slot (or its sink)."""
        n = self.n_sink if sink else self.n_cur
        st = lib.ispa_kv_write(self.handle, layer, ISPA_KV_SINK if sink else ISPA_KV_CURRENT,
                               self._rows(k, n, "k"), self._rows(v, n, "v"), _stream(stream))
        self._check("ispa_kv_write", st)

    def advance(self) -> None:
        self._check("ispa_kv_advance", lib.ispa_kv_advance(self.handle))

    def evict_history(self, layer: int, *, stream=None) -> None:
        self._check("ispa_kv_evict_history",
                    lib.ispa_kv_evict_history(self.handle, layer, _stream(stream)))

    def restore_history(self, layer: int) -> None:
        self._check("ispa_kv_restore_history", lib.ispa_kv_restore_history(self.handle, layer))

    def resident_bytes(self) -> int:
        return int(lib.ispa_kv_resident_bytes(self.handle))

    def attn(self, layer: int, q, sm_scale: float, *, o_local=None, lse_local=None, o_hist=None,
             lse_hist=None, o_full=None, lse_full=None, d_out=None, stream=None) -> None:
        bf, f32 = torch.bfloat16, torch.float32
        n_q = q.shape[0]
        h = self.n_heads * self.head_dim
        if tuple(q.shape) != (n_q, self.n_heads, self.head_dim):
            raise ValueError("q: shape mismatch")
        for name, t in (("o_local", o_local), ("o_hist", o_hist), ("o_full", o_full),
                        ("d_out", d_out)):
            if t is not None and tuple(t.shape) != (n_q, h):
                raise ValueError(f"{name}: expected shape {(n_q, h)}")
        for name, t in (("lse_local", lse_local), ("lse_hist", lse_hist), ("lse_full", lse_full)):
            if t is not None and tuple(t.shape) != (self.n_heads, n_q):
                raise ValueError(f"{name}: expected shape {(self.n_heads, n_q)}")
        st = lib.ispa_kv_attn(
            self.handle, layer, _ptr(q, bf, "q"), n_q, float(sm_scale),
            _ptr(o_local, bf, "o_local"), _ptr(lse_local, f32, "lse_local"),
            _ptr(o_hist, bf, "o_hist"), _ptr(lse_hist, f32, "lse_hist"),
            _ptr(o_full, bf, "o_full"), _ptr(lse_full, f32, "lse_full"),
            _ptr(d_out, bf, "d_out"), _stream(stream))
        _check("ispa_kv_attn", st)

    def layer_forward(self, layer: int, q, sm_scale: float, wo, o_tmp, y, *, stream=None) -> None:
        """y [n_q, h] = attention of the layer (local for an L-layer, full
        otherwise) projected through wo [h, h]; o_tmp [n_q, h] receives O."""
        bf = torch.bfloat16
        n_q = q.shape[0]
        h = self.n_heads * self.head_dim
        if tuple(q.shape) != (n_q, self.n_heads, self.head_dim) or tuple(wo.shape) != (h, h) or \
                tuple(o_tmp.shape) != (n_q, h) or tuple(y.shape) != (n_q, h):
            raise ValueError("layer_forward: shape mismatch")
        st = lib.ispa_kv_layer_forward(self.handle, layer, _ptr(q, bf, "q"), n_q,
                                       float(sm_scale), _ptr(wo, bf, "wo"),
                                       _ptr(o_tmp, bf, "o_tmp"), _ptr(y, bf, "y"),
                                       _stream(stream))
        _check("ispa_kv_layer_forward", st)


def ispa_drift_workspace_bytes(n_layers: int, h: int, n_sample: int) -> int:
    return int(lib.ispa_drift_workspace_bytes(n_layers, h, n_sample))


def ispa_drift_prepare(G, lam: float, n_warm: int, linv, ref, info, workspace, *,
                       stream=None) -> None:
    """G [L, h, h] fp32 -> linv [L, h, h] fp32, ref [L] fp64, info [L] int32."""
    n_layers, h, _ = G.shape
    st = lib.ispa_drift_prepare(n_layers, h, _ptr(G, torch.float32, "G"), float(lam), int(n_warm),
                                _ptr(linv, torch.float32, "linv"),
                                _ptr(ref, torch.float64, "ref"), _ptr(info, torch.int32, "info"),
                                _ptr(workspace, None, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_drift_prepare", st)


def ispa_drift_prepare_factored(n_layers: int, h: int, lam: float, n_warm: int, linv, ref,
                                ridge_workspace, *, stream=None) -> None:
    """linv and ref as ispa_drift_prepare gives them, from the factor the
    preceding ispa_ridge_solve left in ridge_workspace (same G and lambda,
    nothing else run on that workspace in between)."""
    if tuple(linv.shape) != (n_layers, h, h) or ref.shape[0] != n_layers:
        raise ValueError("ispa_drift_prepare_factored: shape mismatch")
    st = lib.ispa_drift_prepare_factored(n_layers, h, float(lam), int(n_warm),
                                         _ptr(linv, torch.float32, "linv"),
                                         _ptr(ref, torch.float64, "ref"),
                                         _ptr(ridge_workspace, None, "workspace"),
                                         ridge_workspace.numel() * ridge_workspace.element_size(),
                                         _stream(stream))
    _check("ispa_drift_prepare_factored", st)


def ispa_drift_score(linv, ref, x, stride: int, score, workspace, *, stream=None) -> None:
    """x [L, n_tok, h] (or [n_tok, h]) bf16 -> score [L] fp64."""
    if x.dim() == 2:
        x = x.unsqueeze(0)
    n_layers, n_tok, h = x.shape
    if tuple(linv.shape) != (n_layers, h, h) or ref.shape[0] != n_layers or \
            score.shape[0] != n_layers:
        raise ValueError("ispa_drift_score: shape mismatch")
    st = lib.ispa_drift_score(n_layers, h, _ptr(linv, torch.float32, "linv"),
                              _ptr(ref, torch.float64, "ref"), _ptr(x, torch.bfloat16, "x"),
                              n_tok, int(stride), _ptr(score, torch.float64, "score"),
                              _ptr(workspace, None, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_drift_score", st)


class Session:
    """ISPA streaming session (ispa_session_* in include/ispa.h): warmup,
    absorption and streaming of all layers over one KV cache, with
    event-triggered recalibration. wo [L, h, h] bf16 holds the original
    weights (kept unchanged); the session owns the active weights and its
    workspace as torch tensors."""

    def __init__(self, wo, *, n_heads: int, head_dim: int, n_sink: int, n_cur: int,
                 hist_capacity: int, k_select: int, t_warm: int, sm_scale: float, lam: float,
                 drift_threshold: float = 0.0, drift_stride: int = 1, flags: int = 0,
                 stream=None):
        n_layers = wo.shape[0]
        self.cfg = SessionConfig(n_layers, n_heads, head_dim, k_select, t_warm, flags, n_sink,
                                 n_cur, hist_capacity, sm_scale, lam, drift_threshold,
                                 drift_stride)
        nbytes = int(lib.ispa_session_workspace_bytes(ct.byref(self.cfg)))
        if nbytes == 0:
            raise IspaError("ispa_session_workspace_bytes", ISPA_ERR_SHAPE)
        self.wo = wo
        self.w_active = torch.empty_like(wo)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=wo.device)
        self.n_layers, self.n_cur = n_layers, n_cur
        self.h = n_heads * head_dim
        h = _p()
        self._h = _p()
        st = lib.ispa_session_create(ct.byref(self.cfg), _ptr(wo, torch.bfloat16, "wo"),
                                     _ptr(self.w_active, torch.bfloat16, "w_active"),
                                     _ptr(self.workspace, None, "workspace"), nbytes,
                                     _stream(stream), ct.byref(h))
        if st != ISPA_OK:
            raise IspaError("ispa_session_create", st, lib.ispa_kv_last_error(None).decode())
        self._h = h
        cache = KVCache.__new__(KVCache)
        cache._h = _p(lib.ispa_session_cache(h))
        cache.n_layers, cache.n_heads, cache.head_dim = n_layers, n_heads, head_dim
        cache.n_sink, cache.n_cur, cache.hist_capacity = n_sink, n_cur, hist_capacity
        cache.close = lambda: None          # owned by the session
        self.cache = cache

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("Session is closed")
        return self._h.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            st = lib.ispa_session_destroy(self._h)
            self._h = _p()
            self.cache._h = _p()
            _check("ispa_session_destroy", st)

    def __del__(self):  # pragma: no cover - depends on collection order
        try:
            self.close()
        except Exception:
            pass

    def layer(self, layer: int, q, y, *, stream=None) -> None:
        if tuple(y.shape) != (self.n_cur, self.h) or q.shape[0] != self.n_cur:
            raise ValueError("Session.layer: shape mismatch")
        st = lib.ispa_session_layer(self.handle, layer, _ptr(q, torch.bfloat16, "q"),
                                    _ptr(y, torch.bfloat16, "y"), _stream(stream))
        if st != ISPA_OK:
            raise IspaError("ispa_session_layer", st, lib.ispa_kv_last_error(self.cache._h).decode())

    def end_chunk(self, *, stream=None) -> int:
        ev = _i(0)
        st = lib.ispa_session_end_chunk(self.handle, _stream(stream), ct.byref(ev))
        if st != ISPA_OK:
            raise IspaError("ispa_session_end_chunk", st,
                            lib.ispa_kv_last_error(self.cache._h).decode())
        return int(ev.value)

    def state(self):
        """(SessionState, is_local list, eps_rel list, drift list)."""
        st = SessionState()
        L = self.n_layers
        loc, eps, dr = (ct.c_int * L)(), (ct.c_double * L)(), (ct.c_double * L)()
        _check("ispa_session_query", lib.ispa_session_query(
            self.handle, ct.byref(st), ct.cast(loc, _p), ct.cast(eps, _p), ct.cast(dr, _p)))
        return st, list(loc), list(eps), list(dr)


def ispa_quantize_fp8(a, q, scale, *, stream=None) -> None:
    """a [rows, k] bf16 -> q [rows, k] uint8 E4M3 codes, scale [rows] fp32."""
    rows, k = a.shape
    if tuple(q.shape) != (rows, k) or tuple(scale.shape) != (rows,):
        raise ValueError("ispa_quantize_fp8: shape mismatch")
    st = lib.ispa_quantize_fp8(_ptr(a, torch.bfloat16, "a"), rows, k, _ptr(q, torch.uint8, "q"),
                               _ptr(scale, torch.float32, "scale"), _stream(stream))
    _check("ispa_quantize_fp8", st)


def ispa_project_w8a8_workspace_bytes(n: int, h_in: int) -> int:
    return int(lib.ispa_project_w8a8_workspace_bytes(n, h_in))


def ispa_project_w8a8(x, wq, w_scale, y, workspace, *, stream=None) -> None:
    """y [n, h_out] bf16 = X W^T with X = x [n, h_in] bf16 quantized per
    token and W = wq [h_out, h_in] E4M3 codes (uint8) with w_scale [h_out]."""
    n, h_in = x.shape
    h_out = wq.shape[0]
    if wq.shape[1] != h_in or tuple(w_scale.shape) != (h_out,) or tuple(y.shape) != (n, h_out):
        raise ValueError("ispa_project_w8a8: shape mismatch")
    st = lib.ispa_project_w8a8(_ptr(x, torch.bfloat16, "x"), _ptr(wq, torch.uint8, "wq"),
                               _ptr(w_scale, torch.float32, "w_scale"),
                               _ptr(y, torch.bfloat16, "y"), n, h_in, h_out,
                               _ptr(workspace, None, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ispa_project_w8a8", st)


def ispa_project_w8a8_noalloc(x, wq, w_scale, y, *, stream=None) -> None:
    """ispa_project_w8a8 with the quantized tokens staged in the library's
    fixed per-device scratch instead of a workspace: allocates nothing. At most
    NOALLOC_MAX_TOKENS rows and NOALLOC_MAX_CODE_BYTES bytes of codes (n * h_in);
    calls that overlap on one GPU race on its scratch."""
    n, h_in = x.shape
    h_out = wq.shape[0]
    if wq.shape[1] != h_in or tuple(w_scale.shape) != (h_out,) or tuple(y.shape) != (n, h_out):
        raise ValueError("ispa_project_w8a8_noalloc: shape mismatch")
    st = lib.ispa_project_w8a8_noalloc(_ptr(x, torch.bfloat16, "x"), _ptr(wq, torch.uint8, "wq"),
                                       _ptr(w_scale, torch.float32, "w_scale"),
                                       _ptr(y, torch.bfloat16, "y"), n, h_in, h_out,
                                       _stream(stream))
    _check("ispa_project_w8a8_noalloc", st)


def ispa_session_layer_grouped(sessions, layer: int, qs, ys, *, stream=None) -> None:
    """The same layer of several Session objects in grouped launches (the
    results equal separate Session.layer calls)."""
    n = len(sessions)
    if not 1 <= n <= MAX_GROUP or len(qs) != n or len(ys) != n:
        raise ValueError(f"ispa_session_layer_grouped: 1..{MAX_GROUP} sessions")
    hs = (_p * n)(*[sess.handle for sess in sessions])
    qp = (_p * n)(*[_ptr(q, torch.bfloat16, "q") for q in qs])
    yp = (_p * n)(*[_ptr(y, torch.bfloat16, "y") for y in ys])
    st = lib.ispa_session_layer_grouped(hs, n, layer, qp, yp, _stream(stream))
    _check("ispa_session_layer_grouped", st)
