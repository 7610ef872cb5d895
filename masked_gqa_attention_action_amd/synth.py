"""Seeded synthetic inputs for the action-expert layer.

This module only draws numbers and rounds them to bfloat16; it holds none of
the layer's arithmetic.  The oracle, the GPU tests and the benchmark all take
their inputs from here, so both sides see bit-identical values.

Shapes follow the suffix row of the shape table in the OpenDM DM0.5
fast-inference article ("TensorRT+Triton+FlexAttention：OpenDM VLA快速推理加速栈
深度剖析", §2.2): hidden 1024, intermediate 4096, head_dim 256, 8 query and 4 KV
heads.  Prefix buckets (576/704/768/896/1024, or a single 2048) come from §3 of
the same article; chunk sizes 10 (LIBERO) and 50 (base model / RoboTwin) come
from the entry table of the DM05 inference guide (§2).

Values are bfloat16 bit patterns (numpy uint16), made by round-to-nearest-even
from float32 draws of numpy's PCG64 generator.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

H, I, D, HQ, HK = 1024, 4096, 256, 8, 4
ROPE_BASE = 10000.0
EPS = 1e-6
BASE_SEED = 20261203
WEIGHT_STD = 0.02

DEFAULT_BUCKETS = (576, 704, 768, 896, 1024)
LONG_BUCKETS = (2048,)


# --------------------------------------------------------------------------
# bfloat16 bit handling (data representation only)
# --------------------------------------------------------------------------
def bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b) -> np.ndarray:
    return bf16_to_f32(b).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits(a)


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------
WEIGHT_KEYS = ("w_mod1", "b_mod1", "w_qkv", "q_norm", "k_norm", "w_o",
               "w_mod2", "b_mod2", "w_gu", "w_down")


def weight_shapes(h=H, i=I, hq=HQ, hk=HK, d=D):
    return {
        "w_mod1": (3 * h, h), "b_mod1": (3 * h,),
        "w_qkv": ((hq + 2 * hk) * d, h),
        "q_norm": (d,), "k_norm": (d,),
        "w_o": (h, hq * d),
        "w_mod2": (3 * h, h), "b_mod2": (3 * h,),
        "w_gu": (2 * i, h), "w_down": (h, i),
    }


def layer_weights(seed: int, h=H, i=I, hq=HQ, hk=HK, d=D, std=WEIGHT_STD) -> dict:
    """All weights of one layer, N(0, std) each, as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return {k: _normal_bf16(rng, s, std) for k, s in weight_shapes(h, i, hq, hk, d).items()}


# --------------------------------------------------------------------------
# per-request inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Request:
    x: np.ndarray        # [C][H] bf16 bits
    cond: np.ndarray     # [H] bf16 bits
    k_pre: np.ndarray    # [n_layers][HK][P_b][D] bf16 bits
    v_pre: np.ndarray    # [n_layers][HK][P_b][D] bf16 bits
    mask: np.ndarray     # [P_b] uint8, nonzero = visible
    valid_len: int
    pos0: int


def make_mask(rng: np.random.Generator, p_bucket: int, len_lo: int, len_hi: int,
              hole_p: float = 0.0):
    """Visibility mask: rows [0, L) visible, L ~ U{len_lo..len_hi}; inside [0, L)
    each row is independently made invisible with probability hole_p."""
    L = int(rng.integers(len_lo, len_hi + 1))
    m = np.zeros(p_bucket, dtype=np.uint8)
    m[:L] = 1
    if hole_p > 0.0:
        holes = rng.random(L) < hole_p
        m[:L][holes] = 0
    return m, L


def make_request(seed: int, chunk: int, p_bucket: int, len_lo: int, len_hi: int,
                 n_layers: int = 1, hole_p: float = 0.0, h=H, hk=HK, d=D,
                 pos0: int | None = None) -> Request:
    rng = np.random.Generator(np.random.PCG64(seed))
    mask, L = make_mask(rng, p_bucket, len_lo, len_hi, hole_p)
    x = _normal_bf16(rng, (chunk, h), 1.0)
    cond = _normal_bf16(rng, (h,), 1.0)
    k_pre = _normal_bf16(rng, (n_layers, hk, p_bucket, d), 1.0)
    v_pre = _normal_bf16(rng, (n_layers, hk, p_bucket, d), 1.0)
    return Request(x=x, cond=cond, k_pre=k_pre, v_pre=v_pre, mask=mask, valid_len=L,
                   pos0=p_bucket if pos0 is None else pos0)


def time_embedding(t: float, h=H) -> np.ndarray:
    """Harness-only conditioning vector for diffusion time t in [0, 1]:
    sin/cos of t*1000 at geometric frequencies (the pages give no formula;
    both sides receive the same vector).  Returned as bf16 bits."""
    half = h // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    a = t * 1000.0 * f
    return bf16_bits(np.concatenate([np.sin(a), np.cos(a)]).astype(np.float32))


def step_times(n_steps: int):
    """t_k = 1 - k / n_steps (harness reading; the pages give 10 steps)."""
    return [1.0 - k / n_steps for k in range(n_steps)]


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    chunk: int
    p_bucket: int
    len_lo: int
    len_hi: int
    hole_p: float
    n_layers: int
    n_steps: int
    config_index: int
    note: str

    @property
    def seed(self) -> int:
        return BASE_SEED + 1000 * self.config_index

    def request_seed(self, b: int) -> int:
        return self.seed + b

    def weight_seed(self, layer: int) -> int:
        return self.seed + 100 + layer


WORKLOADS = {
    # one layer, P=576, last 64 prefix rows invisible, chunk 10 (LIBERO-shaped)
    "c1": Workload("c1", 1, 10, 576, 512, 512, 0.0, 1, 1, 1,
                   "one layer, P_b=576 (rows 512..575 masked), chunk 10"),
    # one layer, P=1024, valid length U{700..1024}, chunk 50
    "c2": Workload("c2", 1, 50, 1024, 700, 1024, 0.0, 1, 1, 2,
                   "one layer, P_b=1024, L~U{700..1024}, chunk 50"),
    # 18-layer stack x 10 denoise steps, P=896 bucket (L in (768, 896])
    "c3": Workload("c3", 1, 50, 896, 769, 896, 0.0, 18, 10, 3,
                   "18 layers x 10 steps, P_b=896, chunk 50, hipGraph"),
    # long prefix 2048 with 5% visibility holes, chunk 50
    "c4": Workload("c4", 1, 50, 2048, 1900, 2048, 0.05, 1, 1, 4,
                   "one layer, P_b=2048, L~U{1900..2048}, 5% holes, chunk 50"),
    # 16 requests, ragged prefixes padded to 1024, chunk 50
    "c5": Workload("c5", 16, 50, 1024, 576, 1024, 0.0, 1, 1, 5,
                   "16 requests, L_b~U{576..1024} in the 1024 bucket, chunk 50"),
    # headline: 18-layer denoise step at P=1024, chunk 50 (c2's mask rule)
    "step1024": Workload("step1024", 1, 50, 1024, 700, 1024, 0.0, 18, 10, 6,
                         "denoise step: 18 layers, P_b=1024, L~U{700..1024}, chunk 50"),
}


def prefix_qkv_inputs(seed: int, tokens: int = 2048, hidden: int = 2560, hq=HQ, hk=HK,
                      d=D, std=WEIGHT_STD):
    """Prefix-side QKV inputs at the Gemma3-4B prefix shape (hidden 2560):
    X [tokens][hidden] N(0,1), W_qkv [(hq+2hk)d][hidden], norm weights [d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return {
        "x": _normal_bf16(rng, (tokens, hidden), 1.0),
        "w_qkv": _normal_bf16(rng, ((hq + 2 * hk) * d, hidden), std),
        "q_norm": _normal_bf16(rng, (d,), std),
        "k_norm": _normal_bf16(rng, (d,), std),
    }


# --------------------------------------------------------------------------
# prefix (prefill) layer inputs, Gemma3-4B shape of the prefix path
# --------------------------------------------------------------------------
PREFIX_H, PREFIX_I = 2560, 10240


def prefix_layer_weights(seed: int, h=PREFIX_H, i=PREFIX_I, hq=HQ, hk=HK, d=D, std=WEIGHT_STD) -> dict:
    """One prefix decoder layer's weights as bf16 bits: matrices N(0, std),
    norm weights N(0, std) (the (1 + w) convention)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = {"w_in": (h,), "w_qkv": ((hq + 2 * hk) * d, h), "q_norm": (d,), "k_norm": (d,),
              "w_o": (h, hq * d), "w_post_attn": (h,), "w_pre_ffn": (h,), "w_gu": (2 * i, h),
              "w_down": (h, i), "w_post_ffn": (h,)}
    return {k: _normal_bf16(rng, s, std) for k, s in shapes.items()}


def prefix_inputs(seed: int, tokens: int, valid_len: int, hole_p: float = 0.0, h=PREFIX_H):
    """Prefix-layer input rows x [tokens][h] ~ N(0, 1) (bf16 bits) and the key
    validity [tokens] (uint8): tokens past valid_len are bucket padding, and a
    fraction hole_p of the others are invisible too (token 0 stays valid)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal_bf16(rng, (tokens, h), 1.0)
    valid = (np.arange(tokens) < valid_len).astype(np.uint8)
    if hole_p > 0:
        holes = rng.random(tokens) < hole_p
        holes[0] = False
        valid[holes] = 0
    return x, valid


# --------------------------------------------------------------------------
# denoise sampler
# --------------------------------------------------------------------------
ACTION_DIM = 32


def sampler_weights(seed: int, a=ACTION_DIM, h=H) -> dict:
    """Sampler weights as bf16 bits, scaled so every stage sees O(1) values:
    W_in [h][a] N(0, 1/a) (unit-variance noise in, O(1) rows out); the time
    MLP's W_t1, W_t2 [h][h] N(0, 0.05^2) (conditioning of O(1), like the
    layers' cond); the final modulation W_fmod [2h][h] N(0, 0.02^2) like the
    layers' W_mod; W_out [a][h] N(0, 1/h) (O(1) velocity from a normalised
    row); biases N(0, 0.02^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    spec = {"w_in": ((h, a), 1.0 / math.sqrt(a)), "b_in": ((h,), WEIGHT_STD),
            "w_t1": ((h, h), 0.05), "b_t1": ((h,), WEIGHT_STD),
            "w_t2": ((h, h), 0.05), "b_t2": ((h,), WEIGHT_STD),
            "w_fmod": ((2 * h, h), WEIGHT_STD), "b_fmod": ((2 * h,), WEIGHT_STD),
            "w_out": ((a, h), 1.0 / math.sqrt(h)), "b_out": ((a,), WEIGHT_STD)}
    return {k: _normal_bf16(rng, s, std) for k, (s, std) in spec.items()}


def sampler_noise(seed: int, batch: int, chunk: int, a=ACTION_DIM) -> np.ndarray:
    """Initial action noise [batch][chunk][a], float32 N(0, 1) (the draw the
    sampler starts from is an input of both sides)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((batch, chunk, a)).astype(np.float32)
