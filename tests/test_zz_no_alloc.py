"""The allocation-free W8A8 projection (ispa_project_w8a8_noalloc, for callers
that cannot allocate device memory) against the workspace entry point
ispa_project_w8a8 on the same inputs: bit-identical outputs on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
codes and scales; nothing of them may leak into the second), and sizes
beyond the fixed scratch rejected before any launch."""
import math

import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from kv_cache_absorption_attn_amd import _lib
from tests.gpu_helpers import dev_bf16, log

pytestmark = pytest.mark.gpu


def _noalloc(x, wq, w_scale, y, stream):
    n, h_in = x.shape
    return _lib.lib.ispa_project_w8a8_noalloc(x.data_ptr(), wq.data_ptr(), w_scale.data_ptr(),
                                              y.data_ptr(), n, h_in, wq.shape[0], stream)


def _case(n, h_in, h_out, seed):
    x = dev_bf16(wl.random_bf16((n, h_in), 0.5, seed))
    w = dev_bf16(wl.random_bf16((h_out, h_in), 1.0 / math.sqrt(h_in), seed + 1))
    wq = torch.empty((h_out, h_in), dtype=torch.uint8, device="cuda")
    w_scale = torch.empty(h_out, dtype=torch.float32, device="cuda")
    ispa.ispa_quantize_fp8(w, wq, w_scale)
    return x, wq, w_scale


def test_noalloc_w8a8_matches_workspace_entry_point():
    stream = torch.cuda.current_stream().cuda_stream
    # a 14B chunk (4680 tokens x 5120: 24 MB of codes), then a smaller call
    for n, h_in, h_out, seed in ((4680, 5120, 5120, 71), (777, 1536, 1536, 73)):
        log(f"noalloc w8a8 n={n} h_in={h_in} h_out={h_out}")
        x, wq, w_scale = _case(n, h_in, h_out, seed)
        y_ref = torch.full((n, h_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ispa.ispa_project_w8a8_workspace_bytes(n, h_in), dtype=torch.uint8,
                         device="cuda")
        ispa.ispa_project_w8a8(x, wq, w_scale, y_ref, ws)
        y = torch.full_like(y_ref, float("nan"))
        assert _noalloc(x, wq, w_scale, y, stream) == _lib.ISPA_OK
        torch.cuda.synchronize()
        assert torch.isfinite(y_ref.float()).all()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_rejects_inputs_beyond_the_scratch():
    stream = torch.cuda.current_stream().cuda_stream
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = dummy.data_ptr()
    L = _lib.lib
    too_many_tokens = _lib.NOALLOC_MAX_TOKENS + 1
    assert L.ispa_project_w8a8_noalloc(p, p, p, p, too_many_tokens, 64, 64, stream) == \
        _lib.ISPA_ERR_SCRATCH
    rows = _lib.NOALLOC_MAX_CODE_BYTES // 5120 + 1
    assert L.ispa_project_w8a8_noalloc(p, p, p, p, rows, 5120, 64, stream) == \
        _lib.ISPA_ERR_SCRATCH
    torch.cuda.synchronize()
