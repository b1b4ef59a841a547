"""Seeded synthetic inputs for the 4-bit group-affine MoE FFN layer.

This module only draws random numbers and rounds them to the storage types the
layer consumes (bf16 bit patterns, packed nibble bytes).  It holds none of the
layer's arithmetic: no dequantisation, routing or expert math lives here, so
both the CPU oracle and the HIP path can consume its arrays without sharing any
computation.

Canonical weight format (the input format of both sides):
  codes   uint8  [E][N][K/2]   two 4-bit codes per byte, low nibble = even k
  scales  uint16 [E][N][K/64]  bf16 bit patterns, one per group of 64 along K
  biases  uint16 [E][N][K/64]  bf16 bit patterns
for gate and up (N = I, K = H) and down (N = H, K = I); the shared expert uses
the same layout with a leading dimension of 1 and I replaced by Is.

Workloads (shapes follow the MoE layer of the "Optimizing on-device inference
for Apple Silicon" page, section on the three workload shapes: 256 routed
experts, top-8, one shared expert; 64-weight groups with bf16 scale and bias,
section on dequantising during the matrix multiply):
  tiny          T=64,  H=256,  E=16,  k=2, I=Is=128, every seed 0
  decode        T=1,   H=2048, E=256, k=8, I=Is=512, weights seed 1, x seed 101
  smallrow      T in {2,3,4,5,8}, same layer, x seed 200+T
  prefill512    T=512, same layer, x seed 300, no logit bias
  prefill4096   T=4096 (chunks of 2048), x seed 400, Zipf(1.1) logit bias with
                rank permutation seed 401

Distributions: codes uniform on 0..15 (uniform random bytes), scales
U(0.005, 0.02) and biases U(-0.1, 0.1) drawn in float64, cast to float32 and
then to bf16 (round to nearest even); router weight N(0, 0.02) in float32;
activations N(0, 1) in float64 -> float32 -> bf16.  Draw order inside one
weight seed: router weight, then gate codes/scales/biases for all experts,
then up, then down, then the shared expert's gate, up, down.
"""
from __future__ import annotations

import numpy as np

GROUP = 64

CONFIGS = {
    "tiny": dict(T=64, H=256, E=16, k=2, I=128, Is=128, wseed=0, xseed=0, zipf_seed=None),
    "decode": dict(T=1, H=2048, E=256, k=8, I=512, Is=512, wseed=1, xseed=101, zipf_seed=None),
    "prefill512": dict(T=512, H=2048, E=256, k=8, I=512, Is=512, wseed=1, xseed=300, zipf_seed=None),
    "prefill4096": dict(T=4096, H=2048, E=256, k=8, I=512, Is=512, wseed=1, xseed=400, zipf_seed=401),
}
SMALLROW_TS = (2, 3, 4, 5, 8)
CHUNK = 2048


def smallrow_config(T: int) -> dict:
    return dict(T=T, H=2048, E=256, k=8, I=512, Is=512, wseed=1, xseed=200 + T, zipf_seed=None)


def config(name: str) -> dict:
    if name.startswith("smallrow"):
        return smallrow_config(int(name[len("smallrow"):]))
    return dict(CONFIGS[name])


# ---- storage-type rounding (not part of the layer's arithmetic) -------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_uniform(rng, lo, hi, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def _qmatrix(rng, E, N, K) -> dict:
    assert K % GROUP == 0
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = _bf16_uniform(rng, 0.005, 0.02, (E, N, K // GROUP))
    biases = _bf16_uniform(rng, -0.1, 0.1, (E, N, K // GROUP))
    return dict(codes=codes, scales=scales, biases=biases)


def gen_weights(H: int, E: int, I: int, Is: int, seed: int) -> dict:
    rng = np.random.default_rng(seed)
    w = dict(H=H, E=E, I=I, Is=Is)
    w["router_w"] = rng.normal(0.0, 0.02, size=(E, H)).astype(np.float32)
    w["gate"] = _qmatrix(rng, E, I, H)
    w["up"] = _qmatrix(rng, E, I, H)
    w["down"] = _qmatrix(rng, E, H, I)
    if Is > 0:
        w["sh_gate"] = _qmatrix(rng, 1, Is, H)
        w["sh_up"] = _qmatrix(rng, 1, Is, H)
        w["sh_down"] = _qmatrix(rng, 1, H, Is)
    return w


def gen_x(T: int, H: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))


def zipf_logit_bias(E: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank), rank a seeded permutation of 1..E.

    This is the log of a Zipf(s) probability mass up to a constant, which
    skews the routing so that expert loads range from none to several hundred
    rows per 2048-token chunk.
    """
    rng = np.random.default_rng(seed)
    rank = rng.permutation(E).astype(np.float64) + 1.0
    return (-s * np.log(rank)).astype(np.float32)


_WCACHE: dict = {}


def make_case(name: str, cache: bool = True) -> dict:
    """Build one workload: layer weights, activations and optional logit bias."""
    c = config(name)
    key = (c["H"], c["E"], c["I"], c["Is"], c["wseed"])
    if cache and key in _WCACHE:
        w = _WCACHE[key]
    else:
        w = gen_weights(c["H"], c["E"], c["I"], c["Is"], c["wseed"])
        if cache:
            _WCACHE[key] = w
    case = dict(name=name, cfg=c, w=w, k=c["k"], T=c["T"])
    case["x"] = gen_x(c["T"], c["H"], c["xseed"])
    case["bias"] = zipf_logit_bias(c["E"], c["zipf_seed"]) if c["zipf_seed"] is not None else None
    return case


def small_layer(T, H, E, k, I, Is, seed, zipf_seed=None) -> dict:
    """An arbitrary small layer (for edge-case tests)."""
    w = gen_weights(H, E, I, Is, seed)
    c = dict(T=T, H=H, E=E, k=k, I=I, Is=Is, wseed=seed, xseed=seed + 1, zipf_seed=zipf_seed)
    case = dict(name=f"small_{T}_{H}_{E}_{k}_{I}_{Is}_{seed}", cfg=c, w=w, k=k, T=T)
    case["x"] = gen_x(T, H, seed + 1)
    case["bias"] = zipf_logit_bias(E, zipf_seed) if zipf_seed is not None else None
    return case
