"""GPU invariants that need no oracle: each compares the HIP path with itself,
bit for bit.

- Run-to-run determinism: the sort ranks rows by slot with ballots and
  popcounts, and the finalize sums in ascending k without atomics, so two
  calls on the same inputs give the same maps and the same output bits.
- Token-permutation equivariance: every output element is one dot product
  over K in a fixed order, whatever row of a tile its token lands in, so
  permuting the tokens permutes the output rows and nothing else.
- Power-of-two scales: adding 1 to every E8M0 byte of W2 doubles W2 exactly,
  hence Y and the output. Without a clamp, SwiGLU is linear in the up half,
  so adding 1 to the up rows' W13 scale bytes doubles the output too. This
  holds on the W4A8 and W4A4 paths as well: the MX scale of a doubled block
  moves up by one and its codes stay the same.
- Tokens with no local expert (every id outside the local range, or masked
  with -1) give exact zeros; a masked slot gives the same output bits as the
  same slot routed to a local expert with weight 0.

Runs whose row counts differ can take different GEMM2 paths under the
device gate, and the two paths use different MFMA shapes. Such comparisons
force one path on both runs.
"""
import functools

import numpy as np
import pytest
import torch

from workloads import LayerShape, make_inputs

from gpu_util import run, say, to_device

pytestmark = pytest.mark.gpu

INV = [
    LayerShape("inv_decode_b32", T=64, E=64, E_g=64, topk=8, H=512, I=256, B=32),
    LayerShape("inv_ep_zipf_b16", T=96, E=64, E_g=128, topk=8, H=1024, I=128, B=16,
               expert_offset=64, routing="zipf"),
    LayerShape("inv_shared_b32", T=48, E=32, E_g=32, topk=4, H=512, I=256, B=32, S=1),
    LayerShape("inv_prefill_b128", T=512, E=8, E_g=8, topk=2, H=512, I=128, B=128),
    LayerShape("inv_split_long_k", T=40, E=16, E_g=16, topk=4, H=512, I=640, B=32),
    LayerShape("inv_decode_w4a8", T=64, E=64, E_g=64, topk=8, H=512, I=256, B=32, a_dtype="mxfp8"),
    LayerShape("inv_prefill_w4a8", T=512, E=8, E_g=8, topk=2, H=512, I=128, B=128, a_dtype="mxfp8"),
    LayerShape("inv_decode_w4a4", T=64, E=64, E_g=64, topk=8, H=512, I=256, B=32, a_dtype="mxfp4"),
    LayerShape("inv_prefill_w4a4", T=512, E=8, E_g=8, topk=2, H=512, I=384, B=128, a_dtype="mxfp4"),
    # decode GEMM1 pairs past one resident round run as K halves: LDS token
    # tiles, per-wave tokens, and the W4A8 kernel
    LayerShape("inv_leftover_tl", T=512, E=64, E_g=64, topk=8, H=512, I=256, B=16),
    LayerShape("inv_leftover_sparse", T=64, E=512, E_g=512, topk=8, H=512, I=256, B=16),
    LayerShape("inv_leftover_w4a8", T=64, E=1024, E_g=1024, topk=16, H=2048, I=256, B=16,
               a_dtype="mxfp8"),
]
FORCES = ["auto", "split", "dense"]
SEED = 4242


@functools.lru_cache(maxsize=None)
def _inputs(name: str) -> dict:
    s = next(v for v in INV if v.name == name)
    return make_inputs(s, SEED + INV.index(s))


def _bits(out: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy()


def _vals(out: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _forward(s: LayerShape, inp: dict, force: str = "auto") -> torch.Tensor:
    out, _ = run(s, to_device(s, inp), force)
    return out


@pytest.mark.parametrize("force", FORCES)
@pytest.mark.parametrize("s", INV, ids=lambda s: s.name)
def test_run_to_run_determinism(s, force):
    say(f"[invariant] determinism {s.name} force={force}")
    inp = _inputs(s.name)
    dev = to_device(s, inp)
    a, _ = run(s, dev, force)
    b, _ = run(s, dev, force)
    assert np.array_equal(_bits(a), _bits(b)), f"{s.name}/{force}: outputs differ between calls"


@pytest.mark.parametrize("force", FORCES)
@pytest.mark.parametrize("s", INV, ids=lambda s: s.name)
def test_token_permutation_equivariance(s, force):
    say(f"[invariant] permutation {s.name} force={force}")
    inp = _inputs(s.name)
    perm = np.random.default_rng(SEED).permutation(s.T)
    pin = dict(inp)
    for k in ("x", "logits", "shared"):
        pin[k] = np.ascontiguousarray(inp[k][perm])
    base = _bits(_forward(s, inp, force))
    got = _bits(_forward(s, pin, force))
    assert np.array_equal(got, base[perm]), f"{s.name}/{force}: permuted output rows differ"


@pytest.mark.parametrize("s", INV, ids=lambda s: s.name)
def test_power_of_two_scale_bytes(s):
    say(f"[invariant] scale bytes {s.name}")
    assert s.swiglu_limit <= 0 and s.activation == "swiglu"
    inp = _inputs(s.name)
    assert int(inp["s2"].max()) < 254 and int(inp["s13"].max()) < 254
    base = _vals(_forward(s, inp))
    assert np.any(base != 0)
    s2 = dict(inp)
    s2["s2"] = inp["s2"] + np.uint8(1)
    assert np.array_equal(_vals(_forward(s, s2)), 2.0 * base), f"{s.name}: s2 + 1 did not double"
    up = dict(inp)
    up["s13"] = inp["s13"].copy()
    up["s13"][:, s.I:, :] += np.uint8(1)  # rows [I, 2I) are the up projection
    assert np.array_equal(_vals(_forward(s, up)), 2.0 * base), f"{s.name}: up s13 + 1 did not double"


@pytest.mark.parametrize("B", [16, 32, 128])
def test_off_range_tokens_are_exact_zeros(B):
    """Local experts [16, 32) of 32; every token's top 4 lie in [0, 16)."""
    s = LayerShape(f"off_range_b{B}", T=40, E=16, E_g=32, topk=4, H=512, I=128, B=B,
                   expert_offset=16)
    say(f"[invariant] off-range tokens B={B}")
    inp = make_inputs(s, SEED + 100 + B)
    inp["logits"][:, 16:] = np.float32(-1.0e4)
    assert np.all(_vals(_forward(s, inp)) == 0.0)
    ids = s.replace(name=f"masked_b{B}", mode="ids")
    iin = make_inputs(ids, SEED + 200 + B)
    iin["topk_ids"][:] = -1
    assert np.all(_vals(_forward(ids, iin)) == 0.0)


@pytest.mark.parametrize("force", ["split", "dense"])
@pytest.mark.parametrize("a_dtype", ["bf16", "mxfp8", "mxfp4"])
def test_masked_ids_contribute_nothing(force, a_dtype):
    s = LayerShape("masked_ids", T=29, E=16, E_g=40, topk=5, H=512, I=128, B=16,
                   expert_offset=10, mode="ids", a_dtype=a_dtype)
    say(f"[invariant] masked ids force={force} a_dtype={a_dtype}")
    inp = make_inputs(s, SEED + 300)
    mask = np.random.default_rng(SEED).random(inp["topk_ids"].shape) < 0.3
    masked = dict(inp)
    masked["topk_ids"] = np.where(mask, np.int32(-1), inp["topk_ids"]).astype(np.int32)
    zero_w = dict(inp)
    zero_w["topk_ids"] = np.where(mask, np.int32(s.expert_offset + 3), inp["topk_ids"]).astype(np.int32)
    zero_w["topk_w"] = np.where(mask, np.float32(0.0), inp["topk_w"]).astype(np.float32)
    a = _bits(_forward(s, masked, force))
    b = _bits(_forward(s, zero_w, force))
    assert np.array_equal(a, b), f"{force}/{a_dtype}: a masked slot changed the output"
