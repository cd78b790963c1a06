"""Seeded synthetic inputs for the ISPA hot path.

This module only *draws* inputs: shapes, seeds, value distributions and the
rounding of the drawn fp32 values to bf16 storage. It holds none of the
method's arithmetic (no attention, no statistics, no solve), so both the
fp64 CPU oracle and the HIP path can take their inputs from here without
sharing any computation.

Workload shapes follow the ISPA paper ("Towards Memory-Efficient
Autoregressive Video Generation via Instance-Specific Parametric
Absorption"): a streaming chunk of 3 latent frames, one sink frame kept in
the local set (§3.1 item 1), a history that grows with the video (§1), a
warmup of T_warm = 12 latent frames = 4 chunks and a budget of K = x*N layers
(§4.1 "Implementation Details", Table 1 caption). Wan-class head geometry
(1.3B: 12 heads x 128; 14B: 40 heads x 128) and 1560 tokens per latent frame
are the model shapes of the backbones named in §4.1.

Generator: numpy PCG64 seeded by SeedSequence([base_seed, config, layer,
step, tensor]). Values are drawn in fp32 and rounded to bf16 with
round-to-nearest-even, so the GPU and the oracle see the same bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

TOKENS_PER_FRAME = 1560

# tensor ids inside the SeedSequence key
T_Q, T_K_SINK, T_V_SINK, T_K_CUR, T_V_CUR, T_K_HIST, T_V_HIST, T_WO = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload: head geometry, KV segment lengths and warmup schedule."""
    name: str
    config_id: int
    n_layers: int
    n_heads: int
    head_dim: int
    n_q: int
    n_sink: int
    n_cur: int
    hist_per_step: tuple          # history length seen at each warmup step
    lam: float
    k_select: int
    qkv_std: float                # std of Q/K/V entries before bf16 rounding
    wo_std: float                 # std of W_o entries before bf16 rounding
    layer_temperature: bool       # per-layer query temperature in [0.5, 2]

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_steps(self) -> int:
        return len(self.hist_per_step)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def n_hist_max(self) -> int:
        return max(self.hist_per_step)


def _frames(n: int) -> int:
    return n * TOKENS_PER_FRAME


# Tiny case: 2 heads x 64 = hidden 128 (the only reading where hidden 128,
# head_dim 64 and a 128x128 Gram all hold), 64 queries, 32 sink + 96 current
# keys, 256 history keys, 3 warmup steps, lambda 1e-2.
TINY = Workload("tiny", 0, 1, 2, 64, 64, 32, 96, (256, 256, 256), 1e-2, 1,
                1.0 / 8.0, 1.0 / math.sqrt(128.0), False)
# Literal single-head variant of the tiny case (hidden = head_dim = 64).
TINY_1HEAD = Workload("tiny_1head", 10, 1, 1, 64, 64, 32, 96, (256, 256, 256),
                      1e-2, 1, 1.0 / 8.0, 1.0 / 8.0, False)
# 1.3B-class single layer: 12 x 128, 4680 queries (3 frames), sink 1 frame,
# current 3 frames, history 18 frames, 4 warmup steps.
WAN13_LAYER = Workload("wan1.3b_layer", 1, 1, 12, 128, _frames(3), _frames(1),
                       _frames(3), (_frames(18),) * 4, 1e-2, 1, 1.0,
                       1.0 / math.sqrt(1536.0), False)
# 1.3B-class full warmup: 30 layers, history 0 -> 18 frames over 4 steps.
WAN13_WARMUP = Workload("wan1.3b_warmup", 2, 30, 12, 128, _frames(3),
                        _frames(1), _frames(3),
                        tuple(_frames(6 * s) for s in range(4)), 1e-2, 15,
                        1.0, 1.0 / math.sqrt(1536.0), True)
# 14B-class full warmup: 40 layers, 40 x 128, history 0 -> 36 frames.
WAN14_WARMUP = Workload("wan14b_warmup", 3, 40, 40, 128, _frames(3),
                        _frames(1), _frames(3),
                        tuple(_frames(12 * s) for s in range(4)), 1e-2, 20,
                        1.0, 1.0 / math.sqrt(5120.0), True)

# 14B-class long-horizon streaming after absorption: one chunk at the longest
# history of the run, 120 latent frames (the F-layers attend all of it). Used
# for sampled-row parity of the full-only pass; the streaming timing draws its
# own device-side inputs.
WAN14_STREAM = Workload("wan14b_stream", 4, 40, 40, 128, _frames(3), _frames(1), _frames(3),
                        (_frames(120),), 1e-2, 20, 1.0, 1.0 / math.sqrt(5120.0), True)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, TINY_1HEAD, WAN13_LAYER, WAN13_WARMUP,
                                   WAN14_WARMUP)}


def streaming_hist_frames() -> List[int]:
    """History lengths (latent frames) of the long-horizon 14B streaming run:
    36 -> 120 frames in 3-frame chunk steps."""
    return list(range(36, 121, 3))


# --------------------------------------------------------------------------
# bf16 storage rounding of the drawn values (input preparation only)
# --------------------------------------------------------------------------

def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(wl: Workload, layer: int, step: int, tensor: int,
            base_seed: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([base_seed, wl.config_id, layer, step, tensor])
    return np.random.Generator(np.random.PCG64(ss))


def draw_bf16(shape, std: float, rng: np.random.Generator) -> np.ndarray:
    """i.i.d. N(0, std^2) drawn in fp32, rounded to bf16; returned as fp32
    arrays whose values are exactly bf16-representable."""
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return bf16_bits_to_f32(round_to_bf16_bits(x))


def layer_temperatures(wl: Workload, base_seed: int = 0) -> np.ndarray:
    """Per-layer query temperature: log-spaced in [0.5, 2], assigned to layers
    by a seeded permutation (so layers differ in how much history matters)."""
    if not wl.layer_temperature or wl.n_layers == 1:
        return np.ones(wl.n_layers, dtype=np.float64)
    t = np.geomspace(0.5, 2.0, wl.n_layers)
    rng = rng_for(wl, 0xFFFF, 0, 99, base_seed)
    return t[rng.permutation(wl.n_layers)]


@dataclasses.dataclass
class StepInputs:
    """Inputs of one (layer, warmup step): all fp32 arrays with bf16 values.

    q: [n_q, n_heads, d]; k_*/v_*: [n, n_heads, d]."""
    q: np.ndarray
    k_sink: np.ndarray
    v_sink: np.ndarray
    k_cur: np.ndarray
    v_cur: np.ndarray
    k_hist: np.ndarray
    v_hist: np.ndarray


def step_inputs(wl: Workload, layer: int, step: int, base_seed: int = 0,
                n_q: Optional[int] = None, n_hist: Optional[int] = None,
                q_gain: float = 1.0) -> StepInputs:
    """Q for this step, the layer's sink frame, this step's current chunk and
    the layer's history truncated to the length of this step.

    The history of a layer is one seeded buffer; step s sees its first
    hist_per_step[s] rows (history grows as the video unfolds)."""
    nh, d = wl.n_heads, wl.head_dim
    nq = wl.n_q if n_q is None else n_q
    nhist = wl.hist_per_step[step] if n_hist is None else n_hist
    temp = layer_temperatures(wl, base_seed)[layer] * q_gain
    std = wl.qkv_std
    q = draw_bf16((nq, nh, d), std * temp, rng_for(wl, layer, step, T_Q, base_seed))
    ks = draw_bf16((wl.n_sink, nh, d), std, rng_for(wl, layer, 0, T_K_SINK, base_seed))
    vs = draw_bf16((wl.n_sink, nh, d), std, rng_for(wl, layer, 0, T_V_SINK, base_seed))
    kc = draw_bf16((wl.n_cur, nh, d), std, rng_for(wl, layer, step, T_K_CUR, base_seed))
    vc = draw_bf16((wl.n_cur, nh, d), std, rng_for(wl, layer, step, T_V_CUR, base_seed))
    # the full-length history buffer is drawn once per layer, then truncated
    kh = draw_bf16((wl.n_hist_max, nh, d), std,
                   rng_for(wl, layer, 0, T_K_HIST, base_seed))[:nhist]
    vh = draw_bf16((wl.n_hist_max, nh, d), std,
                   rng_for(wl, layer, 0, T_V_HIST, base_seed))[:nhist]
    return StepInputs(q, ks, vs, kc, vc, np.ascontiguousarray(kh),
                      np.ascontiguousarray(vh))


def output_projection(wl: Workload, layer: int, base_seed: int = 0) -> np.ndarray:
    """W_o of one layer in nn.Linear layout [out, in], bf16 values."""
    h = wl.hidden
    return draw_bf16((h, h), wl.wo_std, rng_for(wl, layer, 0, T_WO, base_seed))


def random_bf16(shape, std: float, seed: int) -> np.ndarray:
    """Ad-hoc seeded bf16 tensor for unit tests (not tied to a workload)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7777])))
    return draw_bf16(shape, std, rng)
