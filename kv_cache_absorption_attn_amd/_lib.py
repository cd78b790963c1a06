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

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m kv_cache_absorption_attn_amd.build`")
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
lib.ispa_gram_accumulate.restype = _i
lib.ispa_gram_accumulate.argtypes = [_p, _p, _i64, _i, _i, _p, _p, _p, _i, _p]
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

EXPORTED = ("ispa_status_string", "ispa_version", "ispa_attn_decomp", "ispa_gram_accumulate",
            "ispa_ridge_workspace_bytes", "ispa_ridge_solve", "ispa_layer_score",
            "ispa_apply_dW", "ispa_project")


class IspaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {ispa_status_string(status)} (status {status})")
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


def ispa_attn_decomp(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist, sm_scale: float, *,
                     o_local=None, lse_local=None, o_hist=None, lse_hist=None, o_full=None,
                     lse_full=None, d_out=None, stream=None) -> None:
    """q [n_q, H, d]; k_*/v_* [n, H, d] bf16 (k_hist/v_hist may have n = 0).
    Outputs are preallocated tensors: o_* / d_out [n_q, H*d] bf16, lse_*
    [H, n_q] fp32; pass the ones to produce."""
    bf, f32 = torch.bfloat16, torch.float32
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
    st = lib.ispa_attn_decomp(
        _ptr(q, bf, "q"), n_q, *segs, n_heads, head_dim, float(sm_scale),
        _ptr(o_local, bf, "o_local"), _ptr(lse_local, f32, "lse_local"),
        _ptr(o_hist, bf, "o_hist"), _ptr(lse_hist, f32, "lse_hist"),
        _ptr(o_full, bf, "o_full"), _ptr(lse_full, f32, "lse_full"),
        _ptr(d_out, bf, "d_out"), _stream(stream))
    _check("ispa_attn_decomp", st)


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
