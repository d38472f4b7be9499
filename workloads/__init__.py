"""Seeded synthetic workloads for the fused MXFP4 MoE expert layer.

This module is shared by the tests, the benchmark and the smoke check. It
only draws random inputs and describes layer shapes; it holds none of the
layer's arithmetic (no decoding, routing, sorting, GEMM or activation).

The five named layer shapes follow the workloads the sources run the layer
on: the Kimi-K3.1 TP8 decode shape (896 local experts, top-16, hidden 3584,
inter 384) from "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a
Shape template" (section 1, the removed constants), its EP2 half (section 5,
expert offset), a shared-expert shape (the sigmoid shared-expert append page)
and a 32,768-token long prefill (the device-side GEMM2 gate page).

Every array is drawn with numpy's PCG64 in a fixed order from one seed, so
the same (shape, seed) gives the same bytes on every machine.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = ["LayerShape", "CONFIGS", "make_inputs", "f32_to_bf16_bits", "config_seed"]


@dataclass(frozen=True)
class LayerShape:
    """Shape and input recipe of one MoE layer call.

    T tokens, E local experts (E_g global), topk routed experts per token,
    S shared experts appended after the routed ones, H hidden, I inter.
    B is the per-expert row block (decode chunk, 16/32) or prefill M tile.
    """

    name: str
    T: int
    E: int
    E_g: int
    topk: int
    H: int
    I: int
    B: int
    S: int = 0
    expert_offset: int = 0
    swiglu_limit: float = 0.0  # <= 0 means no clamp (SwiGLU only)
    activation: str = "swiglu"  # "swiglu" or "situ"
    act_beta: float = 4.0  # SiTU gate cap beta
    act_linear_beta: float = 25.0  # SiTU up cap (linear beta)
    shared_scale: float = 1.0
    a_dtype: str = "bf16"  # "bf16" (W4A16) or "mxfp8" (W4A8)
    routing: str = "normal"  # "normal" logits N(0,1), "zipf" skewed logits
    zipf_s: float = 1.1
    shared_sigma: float = 2.0
    exp_lo: int = 118  # E8M0 scale bytes drawn uniformly in [exp_lo, exp_hi]
    exp_hi: int = 127
    mode: str = "logits"  # "logits" (router logits in) or "ids" (ids + weights in)

    @property
    def Ep(self) -> int:
        """Weight slots: local routed experts followed by shared experts."""
        return self.E + self.S

    @property
    def Kp(self) -> int:
        """Columns per token after the shared append."""
        return self.topk + self.S

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


CONFIGS: dict[str, LayerShape] = {
    "tiny": LayerShape("tiny", T=4, E=8, E_g=8, topk=2, H=512, I=128, B=16,
                       exp_lo=120, exp_hi=127),
    "decode": LayerShape("decode", T=64, E=896, E_g=896, topk=16, H=3584, I=384, B=32),
    "decode_ep": LayerShape("decode_ep", T=256, E=448, E_g=896, topk=16, H=3584, I=384,
                            B=16, expert_offset=448, routing="zipf"),
    "shared_clamp": LayerShape("shared_clamp", T=512, E=256, E_g=256, topk=8, H=7168,
                               I=2048, B=32, S=1, swiglu_limit=7.0),
    "prefill": LayerShape("prefill", T=32768, E=896, E_g=896, topk=16, H=3584, I=384,
                          B=128),
}
CONFIG_ORDER = ["tiny", "decode", "decode_ep", "shared_clamp", "prefill"]


def config_seed(name: str) -> int:
    """Seed 1000 + the config's 1-based position."""
    return 1000 + CONFIG_ORDER.index(name) + 1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Used only to materialise bf16 inputs; NaN inputs are never drawn.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def make_inputs(shape: LayerShape, seed: int, *, weights: bool = True) -> dict:
    """Draw every input of one layer call.

    Returns numpy arrays:
      x        uint16 [T, H]        bf16 bits, N(0,1) drawn in fp32 then rounded
      logits   float32 [T, E_g]     N(0,1); "zipf" adds -s*ln(rank_e), rank_e a
                                    seeded permutation of 1..E_g
      shared   uint16 [T, S]        bf16 bits of N(0, shared_sigma) (S > 0)
      w13      uint8 [E+S, 2I, H/2] uniform random bytes (two E2M1 codes each)
      s13      uint8 [E+S, 2I, H/32] E8M0 bytes uniform in [exp_lo, exp_hi]
      w2       uint8 [E+S, H, I/2]
      s2       uint8 [E+S, H, I/32]
    In "ids" mode it also returns topk_ids int32 [T, topk] (the top-k of the
    logits is NOT implied: ids are drawn as distinct uniform global experts)
    and topk_w float32 [T, topk] (positive, summing to about 1).
    """
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    out: dict = {}
    out["x"] = f32_to_bf16_bits(rng.standard_normal((s.T, s.H), dtype=np.float32))
    base = rng.standard_normal((s.T, s.E_g), dtype=np.float32)
    if s.routing == "zipf":
        rank = rng.permutation(s.E_g).astype(np.float64) + 1.0
        out["logits"] = (base.astype(np.float64) - s.zipf_s * np.log(rank)[None, :]).astype(np.float32)
    else:
        out["logits"] = base
    if s.S > 0:
        out["shared"] = f32_to_bf16_bits(
            (rng.standard_normal((s.T, s.S), dtype=np.float32) * np.float32(s.shared_sigma)))
    else:
        out["shared"] = np.zeros((s.T, 0), dtype=np.uint16)
    if s.mode == "ids":
        keys = rng.random((s.T, s.E_g))
        out["topk_ids"] = np.argsort(keys, axis=1)[:, : s.topk].astype(np.int32)
        w = rng.random((s.T, s.topk)).astype(np.float32) + np.float32(0.05)
        out["topk_w"] = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    if weights:
        Ep = s.Ep
        out["w13"] = _bytes(rng, (Ep, 2 * s.I, s.H // 2))
        out["s13"] = rng.integers(s.exp_lo, s.exp_hi + 1, size=(Ep, 2 * s.I, s.H // 32), dtype=np.uint8)
        out["w2"] = _bytes(rng, (Ep, s.H, s.I // 2))
        out["s2"] = rng.integers(s.exp_lo, s.exp_hi + 1, size=(Ep, s.H, s.I // 32), dtype=np.uint8)
    return out
