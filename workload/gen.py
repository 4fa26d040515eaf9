"""Seeded synthetic inputs for the routed-expert forward of an MXFP4 Stable LatentMoE layer.

This module only draws random inputs. It holds none of the layer's arithmetic: no dequantisation,
no routing, no matrix products. Both the HIP path (through tests and the bench) and the CPU oracle
consume exactly the arrays returned here.

Shapes follow the Kimi K3 architecture table (AMD article "Day 0 Kimi-K3 Inference Deployment with
ATOM on AMD Instinct MI355X GPUs", section "Model Architecture": hidden 7168, latent 3584, 896 routed
experts with top-16, 2 shared experts, expert intermediate 3072) and one GPU's TP8 share of it
(same article, section "HBM Usage Under TP8": each expert matrix is split eight ways, so the
per-GPU intermediate is 3072 / 8 = 384; router and latent projections are replicated).

Recipe (every tensor has its own random stream, so drawing a subset gives the same bytes):
  * numpy ``Generator(PCG64)`` seeded from ``SeedSequence(seed).spawn(len(STREAMS))``; tensor
    ``STREAMS[i]`` uses child ``i``.
  * x ~ N(0, 1); dense weights ~ N(0, 1/fan_in) (variance 1/fan_in); drawn in float64 and rounded
    to BF16 by torch's round-to-nearest-even conversion (float64 -> float32 -> bfloat16).
  * MXFP4 codes: uniform random bytes (both nibbles uniform over all 16 codes, -0 included).
    E8M0 scales: uniform integers in [120, 124].
  * Skewed routing: per-expert logit bias b_e = ln p(r_e), with p the Zipf(s=1.1) pmf over ranks
    1..E and r a seeded random permutation of 1..E.
  * Exact ties (full-block workload): a seeded sample of ceil(tie_frac * T) tokens; the ties
    themselves are planted into router logits by the test harness.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

STREAMS = (
    "x", "w_router", "zipf_rank", "w_down", "w_up",
    "gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales",
    "sh_gate", "sh_up", "sh_down", "tie_tokens", "sample",
)

SCALE_LO, SCALE_HI = 120, 124
ZIPF_S = 1.1


@dataclass(frozen=True)
class LayerShape:
    """One workload: token count and layer widths.

    T tokens; H hidden width (input/output width when the latent projections are present);
    Lt latent width; E routed experts; K experts per token; I routed-expert intermediate;
    S shared experts of intermediate Is; has_latent False means the input is already the
    latent (no down/up projection, no shared experts, the router reads the latent).
    """
    name: str
    T: int
    H: int
    Lt: int
    E: int
    K: int
    I: int
    S: int
    Is: int
    has_latent: bool
    routing: str          # "uniform" or "zipf"
    tie_frac: float
    seed: int

    @property
    def Hin(self) -> int:
        """Width of x (and of the router's input)."""
        return self.H if self.has_latent else self.Lt

    def with_tokens(self, T: int, name: str | None = None) -> "LayerShape":
        return replace(self, T=T, name=name or f"{self.name}_T{T}")


SHAPES = {
    # Tiny layer: 64 tokens, 512 -> 256 latent, 8 experts top-2, GLU intermediate 128, 1 shared
    # expert whose intermediate equals the routed one (128).
    "tiny": LayerShape("tiny", 64, 512, 256, 8, 2, 128, 1, 128, True, "uniform", 0.0, 0),
    # One GPU's TP8 share of a K3 layer at decode size, uniform routing.
    "tp8_decode_t64": LayerShape("tp8_decode_t64", 64, 7168, 3584, 896, 16, 384, 2, 384, True,
                                 "uniform", 0.0, 1),
    # Same share at prefill size, Zipf-skewed routing.
    "tp8_prefill_t8192": LayerShape("tp8_prefill_t8192", 8192, 7168, 3584, 896, 16, 384, 2, 384,
                                    True, "zipf", 0.0, 2),
    # Full unsharded expert matrices, input already latent, no shared experts, uniform routing.
    "full_experts_t4096": LayerShape("full_experts_t4096", 4096, 3584, 3584, 896, 16, 3072, 0, 0,
                                     False, "uniform", 0.0, 3),
    # Full block at TP8 share, Zipf routing, 1% of tokens with exact rank-16/17 ties.
    "tp8_block_t16384": LayerShape("tp8_block_t16384", 16384, 7168, 3584, 896, 16, 384, 2, 384,
                                   True, "zipf", 0.01, 4),
}


def _rngs(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def _bf16_bits(a64: np.ndarray) -> np.ndarray:
    """float64 array -> BF16 bit patterns (uint16), via torch's RNE conversions."""
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float64)).to(torch.float32)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal_bf16(rng, shape, var: float) -> np.ndarray:
    return _bf16_bits(rng.standard_normal(shape) * math.sqrt(var))


def _codes(rng, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _scales(rng, shape) -> np.ndarray:
    return rng.integers(SCALE_LO, SCALE_HI + 1, size=shape, dtype=np.uint8)


def zipf_bias(E: int, rng) -> np.ndarray:
    ranks = 1 + rng.permutation(E)
    pmf = np.arange(1, E + 1, dtype=np.float64) ** (-ZIPF_S)
    pmf /= pmf.sum()
    return np.log(pmf[ranks - 1]).astype(np.float32)


def make_inputs(shape: LayerShape, names=None) -> dict:
    """Draw the named tensors (default: all that the shape uses).

    Returned arrays (numpy, C-contiguous):
      x [T, Hin] u16 (bf16 bits); w_router [E, Hin] u16; router_bias [E] f32 or None;
      w_down [Lt, H] u16; w_up [H, Lt] u16;
      gate_codes/up_codes [E, I, Lt/2] u8; gate_scales/up_scales [E, I, Lt/32] u8;
      down_codes [E, Lt, I/2] u8; down_scales [E, Lt, I/32] u8;
      sh_gate/sh_up [S, Is, H] u16; sh_down [S, H, Is] u16.
    """
    s = shape
    rng = _rngs(s.seed)
    want = set(names) if names is not None else None

    def need(n):
        return want is None or n in want

    out: dict = {}
    if need("x"):
        out["x"] = _normal_bf16(rng["x"], (s.T, s.Hin), 1.0)
    if need("w_router"):
        out["w_router"] = _normal_bf16(rng["w_router"], (s.E, s.Hin), 1.0 / s.Hin)
    if need("router_bias"):
        out["router_bias"] = zipf_bias(s.E, rng["zipf_rank"]) if s.routing == "zipf" else None
    if s.has_latent:
        if need("w_down"):
            out["w_down"] = _normal_bf16(rng["w_down"], (s.Lt, s.H), 1.0 / s.H)
        if need("w_up"):
            out["w_up"] = _normal_bf16(rng["w_up"], (s.H, s.Lt), 1.0 / s.Lt)
    for m, (n_rows, k) in (("gate", (s.I, s.Lt)), ("up", (s.I, s.Lt)), ("down", (s.Lt, s.I))):
        if need(f"{m}_codes"):
            out[f"{m}_codes"] = _codes(rng[f"{m}_codes"], (s.E, n_rows, k // 2))
        if need(f"{m}_scales"):
            out[f"{m}_scales"] = _scales(rng[f"{m}_scales"], (s.E, n_rows, k // 32))
    if s.S > 0:
        if need("sh_gate"):
            out["sh_gate"] = _normal_bf16(rng["sh_gate"], (s.S, s.Is, s.H), 1.0 / s.H)
        if need("sh_up"):
            out["sh_up"] = _normal_bf16(rng["sh_up"], (s.S, s.Is, s.H), 1.0 / s.H)
        if need("sh_down"):
            out["sh_down"] = _normal_bf16(rng["sh_down"], (s.S, s.H, s.Is), 1.0 / s.Is)
    return out


def tie_tokens(shape: LayerShape) -> np.ndarray:
    """Sorted token indices that receive an exact rank-16/17 tie (empty if tie_frac == 0)."""
    n = math.ceil(shape.tie_frac * shape.T) if shape.tie_frac > 0 else 0
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _rngs(shape.seed)["tie_tokens"]
    return np.sort(rng.choice(shape.T, size=n, replace=False)).astype(np.int64)


def sample_tokens(shape: LayerShape, n: int) -> np.ndarray:
    """Sorted seeded sample of n distinct token indices (all tokens if n >= T)."""
    if n >= shape.T:
        return np.arange(shape.T, dtype=np.int64)
    rng = _rngs(shape.seed)["sample"]
    return np.sort(rng.choice(shape.T, size=n, replace=False)).astype(np.int64)
