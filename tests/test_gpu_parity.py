"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Integer maps (top-k ids, slot experts, counts, offsets, row order, expanded
index, chunk table, gate word, dense tiles) must match bit for bit; routing
weights to 2e-6 relative; layer outputs to a normalised max-abs of 2e-2 and a
relative L2 of 5e-3. Small shapes are compared element by element over the
whole output; the full-size workloads compare every map and a sample of
tokens computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_weight_expert_amd as moe
from workloads import CONFIGS, CONFIG_ORDER, LayerShape, config_seed, f32_to_bf16_bits, make_inputs

from gpu_util import (bf16_dev, check_maps, check_out, covering_tokens, maps_np, oracle_rows,
                      out_np, run, say, to_device)

pytestmark = pytest.mark.gpu

FORCES = {"auto": -1, "split": 0, "dense": 1}

# Reduced shapes the oracle finishes in seconds; several tiles and ragged tails.
SMALL = [
    CONFIGS["tiny"],
    CONFIGS["tiny"].replace(name="tiny_b32", B=32),
    LayerShape("decode_small", T=64, E=64, E_g=64, topk=8, H=512, I=256, B=32),
    LayerShape("ep_zipf_small", T=96, E=64, E_g=128, topk=8, H=1024, I=128, B=16,
               expert_offset=64, routing="zipf"),
    LayerShape("shared_clamp_small", T=48, E=32, E_g=32, topk=4, H=512, I=256, B=32, S=1,
               swiglu_limit=7.0),
    LayerShape("shared2_b16", T=37, E=24, E_g=24, topk=3, H=1536, I=384, B=16, S=2,
               swiglu_limit=3.0, shared_scale=0.5),
    LayerShape("prefill_small", T=1024, E=16, E_g=16, topk=4, H=512, I=128, B=128),
    LayerShape("prefill_b64", T=300, E=8, E_g=8, topk=2, H=512, I=256, B=64),
    LayerShape("prefill_b256", T=700, E=6, E_g=6, topk=2, H=512, I=128, B=256),
    LayerShape("ids_mode", T=29, E=16, E_g=40, topk=5, H=512, I=128, B=16, expert_offset=10,
               mode="ids"),
    LayerShape("one_token", T=1, E=32, E_g=32, topk=8, H=512, I=128, B=16),
    # split GEMM2 over long K (I > 512): odd step count (one-step ring, per-wave
    # token loads), sparse rows (per-wave token loads), and dense rows with
    # chunks of 17-32 rows (token tiles through LDS, two 16-row sub-tiles)
    LayerShape("split_k_odd", T=40, E=16, E_g=16, topk=4, H=512, I=640, B=32),
    LayerShape("split_sparse", T=8, E=64, E_g=64, topk=4, H=512, I=1024, B=16),
    LayerShape("split_dense_b32", T=64, E=8, E_g=8, topk=2, H=1024, I=1024, B=32, swiglu_limit=5.0),
    # SiTU epilogue (K3.1 constants beta 4, linear beta 25, and other caps) on
    # the decode GEMM1 with and without LDS token tiles and on the tiled GEMM1
    LayerShape("situ_decode", T=64, E=32, E_g=32, topk=8, H=512, I=256, B=32, activation="situ"),
    LayerShape("situ_sparse_b16", T=20, E=64, E_g=64, topk=4, H=1024, I=128, B=16,
               activation="situ", act_beta=2.0, act_linear_beta=8.0),
    LayerShape("situ_prefill", T=1024, E=16, E_g=16, topk=4, H=512, I=128, B=128, S=1,
               activation="situ"),
    # the long-prefill kernels at their own inter size: I = 384 (and 768) is a
    # multiple of 192, so GEMM1 runs 384-row weight tiles, and the dense GEMM2
    # keeps the act tile resident (I <= 384) or takes the generic tiled path;
    # many 128- and 256-row tiles per expert with ragged tails
    LayerShape("prefill_i384_b128", T=2048, E=16, E_g=16, topk=4, H=512, I=384, B=128),
    LayerShape("prefill_i384_b256", T=2048, E=12, E_g=12, topk=4, H=1024, I=384, B=256, S=1,
               swiglu_limit=6.0),
    LayerShape("prefill_i768_b128", T=1536, E=10, E_g=10, topk=4, H=512, I=768, B=128),
    # I = 512: the longest K of the split stream (four steps in registers),
    # with bf16 act outside the one-launch gated GEMM2 (the stream kernel,
    # then the generic tiled dense kernel); decode and 256-row-tile prefill
    LayerShape("i512_decode", T=48, E=16, E_g=16, topk=4, H=512, I=512, B=32),
    LayerShape("i512_prefill_b128", T=1024, E=8, E_g=8, topk=2, H=512, I=512, B=128),
    # decode GEMM1 with LDS token tiles and 16-feature items whose (chunk,
    # feature group) pairs overfill one resident round a little (about 4,600
    # pairs against the 4,096 wave slots of MI355X): the pairs left over run
    # as K halves joined through LDS
    LayerShape("gemm1_leftover_halves", T=512, E=64, E_g=64, topk=8, H=512, I=256, B=16),
    # the same with per-wave token loads (about one row per expert): about
    # 5,150 pairs against one round of 3,072 wave slots, the second round
    # run as K halves whose sums meet in the second wave's scale block
    LayerShape("gemm1_leftover_sparse", T=64, E=512, E_g=512, topk=8, H=512, I=256, B=16),
]


@pytest.mark.parametrize("force", list(FORCES))
@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_small_full_parity(s, force):
    say(f"[small] {s.name} force={force}")
    inp = make_inputs(s, 500 + SMALL.index(s))
    if s.mode == "ids":
        inp["topk_ids"][0, :] = -1
        inp["topk_ids"][1, 0] = 0  # outside the local range [10, 26)
    ref = oracle.reference_forward(s, inp, force_path=FORCES[force])
    dev = to_device(s, inp)
    out, ws = run(s, dev, force)
    check_maps(s, maps_np(s, ws, force), ref)
    check_out(out_np(out), ref["out"], f"{s.name}/{force}")


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([[0, T - 1], extra]))


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_config_parity(name):
    s = CONFIGS[name]
    say(f"[config] {name}: T={s.T} E={s.E}/{s.E_g} topk={s.topk} S={s.S} H={s.H} I={s.I} B={s.B}")
    inp = make_inputs(s, config_seed(name))
    dev = to_device(s, inp)
    ref = oracle.reference_forward(s, inp, compute_out=(name == "tiny"))
    if name == "prefill":
        # rows in every expert's ragged tail chunk and at every position of a
        # 128-row tile, computed by the oracle grouped by expert
        toks = covering_tokens(ref, s.Kp, s.B, 128)
        want = oracle_rows(s, inp, toks)
    elif name in ("decode", "decode_ep"):
        # every token: the oracle finishes these in seconds
        toks = np.arange(s.T)
        want = oracle.sampled_forward(s, inp, toks)
    else:
        toks = _sample_tokens(s.T, 8, 7)
        want = ref["out"][toks] if name == "tiny" else oracle.sampled_forward(s, inp, toks)
    auto_path = ref["gate"][0]
    for force in ("auto", "split" if auto_path == 1 else "dense"):
        say(f"  force={force}")
        out, ws = run(s, dev, force)
        r = ref if force == "auto" else oracle.reference_forward(s, inp, FORCES[force], compute_out=False)
        check_maps(s, maps_np(s, ws, force), r)
        got = out_np(out)
        check_out(got[toks], want, f"{name}/{force} sampled tokens {len(toks)}")
        assert np.all(np.isfinite(got))
        del out, ws
    torch.cuda.empty_cache()


# The decode GEMM1's (chunk, 16-feature group) pairs against one resident
# round (4,096 wave slots on MI355X, 512 pairs per XCD): exactly one round
# (T = 452), a few pairs left over (456), nearly half a round left over (704,
# the most that runs as K halves) and just past it (720, the plain mapping);
# at 456 the last XCD's range is cut short.
@pytest.mark.parametrize("T", [452, 456, 704, 720])
def test_gemm1_leftover_edges(T):
    s = LayerShape(f"gemm1_leftover_T{T}", T=T, E=64, E_g=64, topk=8, H=512, I=256, B=16)
    say(f"[leftover] T={T}")
    inp = make_inputs(s, 900 + T)
    ref = oracle.reference_forward(s, inp)
    dev = to_device(s, inp)
    out, ws = run(s, dev, "auto")
    check_maps(s, maps_np(s, ws, "auto"), ref)
    check_out(out_np(out), ref["out"], s.name)


def test_situ_kimi_decode_shape():
    """The K3.1 TP8 decode shape with its own activation, SiTU(4, 25)."""
    s = CONFIGS["decode"].replace(activation="situ", name="decode_situ")
    say(f"[config] {s.name}")
    inp = make_inputs(s, config_seed("decode"))
    dev = to_device(s, inp)
    ref = oracle.reference_forward(s, inp, compute_out=False)
    toks = np.arange(s.T)  # every token
    out, ws = run(s, dev)
    check_maps(s, maps_np(s, ws), ref)
    check_out(out_np(out)[toks], oracle.sampled_forward(s, inp, toks), f"{s.name} all tokens")
    del out, ws
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def kimi_weights():
    s = CONFIGS["decode"]
    inp = make_inputs(s, 4242)
    return s, inp, to_device(s, inp)


@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("T", [1, 7, 48, 96, 256])
def test_kimi_shape_token_sweep(kimi_weights, T, B):
    base, winp, wdev = kimi_weights
    s = base.replace(T=T, B=B, name=f"sweep_T{T}_B{B}")
    say(f"[sweep] T={T} B={B}")
    tok = make_inputs(s, 9000 + T * 7 + B, weights=False)
    inp = {**winp, "x": tok["x"], "logits": tok["logits"], "shared": tok["shared"]}
    dev = dict(wdev)
    dev["x"] = bf16_dev(inp["x"])
    dev["logits"] = torch.from_numpy(inp["logits"]).cuda()
    ref = oracle.reference_forward(s, inp, compute_out=False)
    out, ws = run(s, dev)
    check_maps(s, maps_np(s, ws), ref)
    toks = _sample_tokens(T, 3, T)
    check_out(out_np(out)[toks], oracle.sampled_forward(s, inp, toks), f"T{T}/B{B}")


# ------------------------------------------------------------------ W4A8
# MXFP8 activations: x's codes and scales bit-exact (the quantiser is exact in
# fp32); the layer output to the same tolerances as W4A16 against the
# quantisation-aware oracle (act is quantised from fp32 on the GPU and from
# fp64 in the oracle, so an act code at a rounding boundary may differ by one).
SMALL_A8 = [
    LayerShape("a8_decode_small", T=64, E=64, E_g=64, topk=8, H=512, I=256, B=32, a_dtype="mxfp8"),
    LayerShape("a8_ep_zipf", T=96, E=64, E_g=128, topk=8, H=1024, I=128, B=16, expert_offset=64,
               routing="zipf", a_dtype="mxfp8"),
    LayerShape("a8_shared_clamp", T=48, E=32, E_g=32, topk=4, H=512, I=384, B=32, S=1,
               swiglu_limit=7.0, a_dtype="mxfp8"),
    LayerShape("a8_prefill_small", T=1024, E=16, E_g=16, topk=4, H=512, I=128, B=128,
               a_dtype="mxfp8"),
    LayerShape("a8_prefill_b256", T=700, E=6, E_g=6, topk=2, H=1536, I=256, B=256, a_dtype="mxfp8"),
    LayerShape("a8_one_token", T=1, E=32, E_g=32, topk=8, H=512, I=128, B=16, a_dtype="mxfp8"),
    LayerShape("a8_situ", T=64, E=16, E_g=16, topk=4, H=512, I=256, B=32, activation="situ",
               a_dtype="mxfp8"),
    LayerShape("a8_situ_prefill", T=700, E=6, E_g=6, topk=2, H=512, I=256, B=128,
               activation="situ", act_beta=3.0, act_linear_beta=10.0, a_dtype="mxfp8"),
    # the W4A8 long-prefill kernels at I = 384: tiled GEMM1 and the resident
    # dense GEMM2 over many 128- and 256-row tiles with ragged tails
    LayerShape("a8_prefill_i384_b128", T=2048, E=16, E_g=16, topk=4, H=512, I=384, B=128,
               a_dtype="mxfp8"),
    LayerShape("a8_prefill_i384_b256", T=2048, E=12, E_g=12, topk=4, H=1024, I=384, B=256, S=1,
               swiglu_limit=6.0, a_dtype="mxfp8"),
    # I = 512, the largest the MX paths take: four K steps in the gated
    # GEMM2's stream and resident bodies, decode and tiled GEMM1
    LayerShape("a8_i512_decode", T=48, E=16, E_g=16, topk=4, H=512, I=512, B=32, a_dtype="mxfp8"),
    LayerShape("a8_i512_prefill_b128", T=1024, E=8, E_g=8, topk=2, H=512, I=512, B=128,
               a_dtype="mxfp8"),
]


def _check_xq(got, ref):
    assert np.array_equal(got["xq"], ref["xq"]), "MXFP8 x codes differ"
    assert np.array_equal(got["xs"], ref["xs"]), "MXFP8 x scales differ"


@pytest.mark.parametrize("force", list(FORCES))
@pytest.mark.parametrize("s", SMALL_A8, ids=lambda s: s.name)
def test_w4a8_small_full_parity(s, force):
    say(f"[w4a8] {s.name} force={force}")
    inp = make_inputs(s, 700 + SMALL_A8.index(s))
    ref = oracle.reference_forward(s, inp, force_path=FORCES[force])
    dev = to_device(s, inp)
    out, ws = run(s, dev, force)
    got = maps_np(s, ws, force)
    check_maps(s, got, ref)
    _check_xq(got, ref)
    check_out(out_np(out), ref["out"], f"{s.name}/{force}")


def test_w4a8_quant_special_values():
    """Zeros, signed zeros, subnormal-range and saturating blocks of x."""
    s = LayerShape("a8_special", T=4, E=4, E_g=4, topk=2, H=512, I=128, B=16, a_dtype="mxfp8")
    inp = make_inputs(s, 77)
    x = inp["x"].copy()
    x[0, :32] = 0                      # all-zero block -> scale 0, codes 0
    x[0, 32:64] = 0x8000               # negative zeros -> codes 0x80
    x[1, :32] = 0x0001                 # bf16 subnormals: scale byte clamps to 0
    x[1, 32:64] = 0x7F00               # huge values (2^127): scale byte 246
    x[2, :32] = np.arange(32, dtype=np.uint16) + 0x3F80  # 1.0 .. just above, ties
    x[3, :32] = 0xC3E0                 # -448 exactly
    x[3, 32:64] = 0x43F8               # 496: saturates to 448 after scaling
    inp["x"] = x
    ref = oracle.reference_forward(s, inp)
    out, ws = run(s, to_device(s, inp))
    _check_xq(maps_np(s, ws), ref)


# ------------------------------------------------------------------ W4A4
# MXFP4 activations (the FP4 path of "SGLang CUTLASS MoE", section 6, in the
# weights' MX block format): x's codes and scales bit-exact; outputs to the
# same tolerances against the quantisation-aware oracle (an act code at an
# E2M1 rounding boundary may land one step apart, since act is quantised
# from fp32 here and from fp64 there).
SMALL_A4 = [s.replace(name=s.name.replace("a8_", "a4_"), a_dtype="mxfp4") for s in SMALL_A8]


@pytest.mark.parametrize("force", list(FORCES))
@pytest.mark.parametrize("s", SMALL_A4, ids=lambda s: s.name)
def test_w4a4_small_full_parity(s, force):
    say(f"[w4a4] {s.name} force={force}")
    inp = make_inputs(s, 800 + SMALL_A4.index(s))
    ref = oracle.reference_forward(s, inp, force_path=FORCES[force])
    dev = to_device(s, inp)
    out, ws = run(s, dev, force)
    got = maps_np(s, ws, force)
    check_maps(s, got, ref)
    _check_xq(got, ref)
    check_out(out_np(out), ref["out"], f"{s.name}/{force}")


def test_w4a4_quant_special_values():
    """Zero, signed-zero, subnormal, saturating and exact-tie blocks of x."""
    s = LayerShape("a4_special", T=6, E=4, E_g=4, topk=2, H=512, I=128, B=16, a_dtype="mxfp4")
    inp = make_inputs(s, 78)
    x = inp["x"].copy()
    x[0, :32] = 0                      # all-zero block -> scale 0, codes 0
    x[0, 32:64] = 0x8000               # negative zeros -> codes 8
    x[1, :32] = 0x0001                 # bf16 subnormals: scale byte clamps to 0
    x[1, 32:64] = 0x7F00               # 2^127: scale byte 252, code 6 (4.0)
    x[2, :32] = np.arange(32, dtype=np.uint16) + 0x3F80  # 1.0 .. just above
    x[3, :32] = 0xC0C0                 # -6 exactly
    x[3, 32:64] = 0x40E0               # 7: saturates to 6 after scaling
    # ties between E2M1 neighbours (amax 5 -> scale 1): 0.25 .. 5.0, both signs
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x[4, :32] = f32_to_bf16_bits(np.resize(np.concatenate([ties, -ties]), 32))
    x[5, :32] = f32_to_bf16_bits(np.resize(np.concatenate([ties, -ties]) * np.float32(2 ** -20), 32))
    inp["x"] = x
    ref = oracle.reference_forward(s, inp)
    out, ws = run(s, to_device(s, inp))
    _check_xq(maps_np(s, ws), ref)


@pytest.mark.parametrize("name", ["decode", "decode_ep", "prefill"])
def test_w4a4_config_parity(name):
    s = CONFIGS[name].replace(a_dtype="mxfp4", name=name + "_w4a4")
    say(f"[w4a4 config] {s.name}")
    inp = make_inputs(s, config_seed(name))
    dev = to_device(s, inp)
    ref = oracle.reference_forward(s, inp, compute_out=False)
    if name == "prefill":
        toks = covering_tokens(ref, s.Kp, s.B, 128)
        want = oracle_rows(s, inp, toks)
    elif name in ("decode", "decode_ep"):  # every token: the oracle finishes these in seconds
        toks = np.arange(s.T)
        want = oracle.sampled_forward(s, inp, toks)
    else:
        toks = _sample_tokens(s.T, 8, 12)
        want = oracle.sampled_forward(s, inp, toks)
    out, ws = run(s, dev)
    got = maps_np(s, ws)
    check_maps(s, got, ref)
    _check_xq(got, ref)
    check_out(out_np(out)[toks], want, f"{s.name} sampled tokens {len(toks)}")
    del out, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode", "decode_ep", "prefill"])
def test_w4a8_config_parity(name):
    s = CONFIGS[name].replace(a_dtype="mxfp8", name=name + "_w4a8")
    say(f"[w4a8 config] {s.name}")
    inp = make_inputs(s, config_seed(name))
    dev = to_device(s, inp)
    ref = oracle.reference_forward(s, inp, compute_out=False)
    if name == "prefill":
        toks = covering_tokens(ref, s.Kp, s.B, 128)
        want = oracle_rows(s, inp, toks)
    elif name in ("decode", "decode_ep"):  # every token: the oracle finishes these in seconds
        toks = np.arange(s.T)
        want = oracle.sampled_forward(s, inp, toks)
    else:
        toks = _sample_tokens(s.T, 8, 11)
        want = oracle.sampled_forward(s, inp, toks)
    out, ws = run(s, dev)
    got = maps_np(s, ws)
    check_maps(s, got, ref)
    _check_xq(got, ref)
    check_out(out_np(out)[toks], want, f"{s.name} sampled tokens {len(toks)}")
    del out, ws
    torch.cuda.empty_cache()


# ------------------------------------------------------------ routing edge cases
@pytest.mark.parametrize("E_g,topk", [(8, 2), (130, 5), (896, 16), (2048, 32)])
def test_routing_ties_and_signed_zeros(E_g, topk):
    """Top-k ids bit-exact under heavy ties (equal logits rank by lower id)
    and with -0.0 and +0.0 logits comparing equal. At most 16 experts are
    local, so most routed slots map to -1 and the GEMMs stay small."""
    s = LayerShape(f"ties_{E_g}", T=96, E=min(16, E_g), E_g=E_g, topk=topk, H=512, I=128, B=16)
    inp = make_inputs(s, 900 + E_g)
    rng = np.random.default_rng(E_g)
    lg = rng.integers(-2, 3, size=(s.T, E_g)).astype(np.float32)  # five distinct values
    lg[0::3] = 0.0
    lg[0::3, ::2] = -0.0                       # rows of signed zeros only
    lg[1::3, :topk // 2 + 1] = np.float32(7.5)  # a tie straddling the top-k boundary
    inp["logits"] = lg
    ref = oracle.reference_forward(s, inp, compute_out=False)
    out, ws = run(s, to_device(s, inp))
    check_maps(s, maps_np(s, ws), ref)


@pytest.mark.parametrize("E_g,topk", [(8, 2), (130, 5), (896, 16), (2048, 32)])
def test_routing_threshold_ties(E_g, topk):
    """Ties among few candidates: a group of equal logits straddles the top-k
    boundary while the rest of the row stays distinct (the selection ranks
    the keys at or above a threshold, ties by lower id); groups spread over
    ids that fall in different lanes and lane slots; a group tied with the
    row's own maximum; signed zeros as the top values; rows where many keys
    tie at the threshold (the round-based selection)."""
    s = LayerShape(f"thr_ties_{E_g}", T=64, E=min(16, E_g), E_g=E_g, topk=topk, H=512, I=128, B=16)
    inp = make_inputs(s, 980 + E_g)
    lg = inp["logits"].copy()
    rng = np.random.default_rng(E_g + 7)
    g = min(topk + 3, E_g)
    for t in range(s.T):
        ids = rng.choice(E_g, size=g, replace=False)
        if t % 4 == 0:
            lg[t, ids] = np.float32(9.0)                         # above every other logit
        elif t % 4 == 1:
            lg[t, ids] = lg[t].max()                             # tied with the row's maximum
        elif t % 4 == 2:
            lg[t] = -np.abs(lg[t]) - np.float32(1.0)             # all below zero, then
            lg[t, ids] = np.where(np.arange(g) % 2 == 0, np.float32(0.0), np.float32(-0.0))
        else:
            lg[t, : max(E_g // 2, topk)] = np.float32(3.0)        # many equal at the threshold
    inp["logits"] = lg
    ref = oracle.reference_forward(s, inp, compute_out=False)
    out, ws = run(s, to_device(s, inp))
    check_maps(s, maps_np(s, ws), ref)


@pytest.mark.parametrize("E_g,topk", [(130, 5), (896, 16)])
def test_routing_non_finite_logits(E_g, topk):
    """NaN logits rank below -inf (ties by lower id) and a selected NaN gets
    weight 0; infinities follow IEEE arithmetic (a selected +inf, or an
    all -inf selection, makes the token's weights NaN). Ids bit-exact,
    weights equal including their NaN positions."""
    s = LayerShape(f"nonfinite_{E_g}", T=64, E=16, E_g=E_g, topk=topk, H=512, I=128, B=16)
    inp = make_inputs(s, 950 + E_g)
    lg = inp["logits"].copy()
    rng = np.random.default_rng(E_g + 1)
    lg[0::4][rng.random(lg[0::4].shape) < 0.3] = np.nan   # scattered NaNs
    lg[1] = np.nan                                          # all NaN
    lg[2, :] = np.nan
    lg[2, E_g - topk // 2:] = 1.0                           # fewer numbers than topk
    lg[3, ::3] = -np.inf                                    # -inf among numbers
    lg[5, :] = -np.inf                                      # all -inf
    lg[6, 7] = np.inf                                       # one +inf
    lg[7, 1::2] = np.inf                                    # many +inf, ties
    lg[9, :topk + 3] = -np.inf
    lg[9, topk + 3:] = np.nan                               # -inf before NaN
    inp["logits"] = lg
    ref = oracle.reference_forward(s, inp, compute_out=False)
    out, ws = run(s, to_device(s, inp))
    check_maps(s, maps_np(s, ws), ref)


# Slot counts above the single-block sort (8192 slots): the multi-kernel sort
# (per-range counts, scan + gate, scatter), with a ragged last range, a range
# count that is not a multiple of 4, and skewed routing.
@pytest.mark.parametrize("s", [
    LayerShape("sort_ragged", T=3001, E=40, E_g=48, topk=4, H=512, I=128, B=64, expert_offset=4),
    LayerShape("sort_zipf", T=2500, E=96, E_g=96, topk=8, H=512, I=128, B=128, routing="zipf"),
    LayerShape("sort_many", T=4097, E=300, E_g=300, topk=6, H=512, I=128, B=32, S=1),
], ids=lambda s: s.name)
def test_large_sort_maps(s):
    say(f"[large sort] {s.name}: {s.T * s.Kp} slots")
    inp = make_inputs(s, 321)
    for force in ("auto", "split", "dense"):
        ref = oracle.reference_forward(s, inp, force_path=FORCES[force], compute_out=False)
        out, ws = run(s, to_device(s, inp), force)
        check_maps(s, maps_np(s, ws, force), ref)
        toks = _sample_tokens(s.T, 4, 5)
        check_out(out_np(out)[toks], oracle.sampled_forward(s, inp, toks), f"{s.name}/{force}")


# The largest supported sizes: H = I = 8192 (the longest K loops and the
# largest LDS scale blocks) on the decode, split, tiled and generic dense
# GEMM paths, and E + S = 2048 local experts through both sort paths.
@pytest.mark.parametrize("s", [
    LayerShape("max_hi_decode", T=9, E=2, E_g=2, topk=2, H=8192, I=8192, B=16),
    LayerShape("max_hi_prefill", T=160, E=2, E_g=2, topk=1, H=8192, I=8192, B=128),
    LayerShape("max_experts_small_sort", T=200, E=2047, E_g=2047, topk=32, H=512, I=128, B=32, S=1),
    LayerShape("max_experts_large_sort", T=300, E=2047, E_g=2047, topk=32, H=512, I=128, B=16, S=1),
], ids=lambda s: s.name)
def test_maximum_sizes(s):
    say(f"[max] {s.name}: {s.T * s.Kp} slots, H={s.H} I={s.I} E'={s.Ep}")
    inp = make_inputs(s, 4321)
    dev = to_device(s, inp)
    toks = _sample_tokens(s.T, 2, 9)
    want = oracle.sampled_forward(s, inp, toks)  # the same under every GEMM2 path
    for force in ("auto", "split", "dense"):
        ref = oracle.reference_forward(s, inp, force_path=FORCES[force], compute_out=False)
        out, ws = run(s, dev, force)
        check_maps(s, maps_np(s, ws, force), ref)
        check_out(out_np(out)[toks], want, f"{s.name}/{force}")
        del out, ws
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("rows,row_bytes", [(16, 64), (48, 192), (256, 1792), (768, 1792)])
def test_prepack_layout(rows, row_bytes):
    """Prepacked weights: block (row group g, K step k) holds rows 16g..16g+15,
    bytes 64k..64k+63 of the row-major matrix, row-major inside the block."""
    rng = np.random.default_rng(rows + row_bytes)
    w = rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)
    got = moe.prepack(torch.from_numpy(w).cuda()).cpu().numpy().reshape(-1)
    want = w.reshape(rows // 16, 16, row_bytes // 64, 64).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(got, want)


def test_row_major_weight_tag_rejected_before_launch():
    """A forward call whose shape tags w13/w2 as row-major fails with
    MOE_ERR_UNSUPPORTED and enqueues nothing: out and the workspace keep
    their contents."""
    s = CONFIGS["tiny"]
    inp = make_inputs(s, 31)
    dev = to_device(s, inp)
    shp = moe.Shape(T=s.T, E=s.E, E_global=s.E_g, topk=s.topk, H=s.H, I=s.I, block_n=s.B,
                    weight_layout="row_major")
    ws = torch.full((moe.query(shp),), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full((s.T, s.H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(dev["x"], dev["w13"], dev["s13"], dev["w2"], dev["s2"], shp,
                    router_logits=dev["logits"], out=out, workspace=ws)
    assert ei.value.code == 2
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0)) and bool(torch.all(ws == 0x5A))
