"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against one of: a value the source pages print
(golden files under tests/golden, each citing its page), a closed form, a
library routine (torch's float8 dtypes, scipy), an invariant, or brute force
on tiny inputs. The last group plants mistakes in the oracle and checks that
a pin catches each one.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import mx as omx
from oracle import moe as omoe
from workloads import LayerShape, make_inputs, f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _e2m1_table():
    rows = _golden_rows("e2m1_codes.txt")
    return np.array([float(r[2]) for r in sorted(rows, key=lambda r: int(r[0]))])


# ----------------------------------------------------------------- formats

def test_e2m1_decode_matches_golden_table():
    want = _e2m1_table()
    got = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # code 8 is -0.0


def test_e2m1_largest_magnitude_and_order():
    mags = oracle.e2m1_decode(np.arange(8))
    assert mags.max() == 6.0  # FLOAT4_E2M1_MAX
    assert np.all(np.diff(mags) > 0)
    assert np.array_equal(oracle.e2m1_decode(np.arange(8, 16)), -mags)


def test_e8m0_decode_matches_torch_float8_e8m0fnu():
    b = torch.arange(256, dtype=torch.uint8)
    want = b.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = oracle.e8m0_decode(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255], want[:255])


def test_dequant_nibble_order_and_scale_groups():
    # One row of K = 64: byte j holds elements 2j (low nibble) and 2j+1 (high).
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x72      # element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    packed[0, 16] = 0xA5     # element 32 = code 5 (3.0), element 33 = code 10 (-1.0)
    scales = np.array([[127, 129]], np.uint8)  # group 0 x1, group 1 x4
    w = oracle.dequant_mxfp4(packed, scales)[0]
    assert w[0] == 1.0 and w[1] == 6.0
    assert w[32] == 12.0 and w[33] == -4.0
    assert np.count_nonzero(w) == 4


def test_mxfp4_values_exact_in_bf16():
    # Every E2M1 value times 2^(e-127), e in [0, 252], is a bf16 number: the
    # basis for decoding weights to bf16 without rounding.
    vals = oracle.e2m1_decode(np.arange(16))[:, None] * np.ldexp(1.0, np.arange(0, 253) - 127)[None, :]
    t = torch.from_numpy(vals.ravel())
    assert torch.equal(t.to(torch.bfloat16).double(), t)


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    want = b.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 40,
        rng.standard_normal(5000) * 1e-2,          # subnormal range
        oracle.e4m3_decode(np.arange(126)) * 1.0,  # exact codes
        # midpoints between neighbouring codes: ties to even
        0.5 * (oracle.e4m3_decode(np.arange(0, 125)) + oracle.e4m3_decode(np.arange(1, 126))),
        [448.0, 455.0, 463.9, 1e6, -1e6, 0.0],
    ])
    v = np.concatenate([v, -v])
    got = omx._e4m3_encode(v)
    clamped = np.clip(v, -448.0, 448.0)
    want = torch.from_numpy(clamped).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_mxfp8_shared_exponent_worked_examples():
    blk = np.zeros((4, 32))
    blk[0, 5] = 1.0      # amax 1 -> shared exponent -8 -> byte 119; 1.0 -> 256 = code 0x78
    blk[1, :] = 448.0    # amax 448 -> exponent 0 -> byte 127; 448 -> code 0x7E
    blk[2, 3] = -500.0   # amax 500 -> exponent 0; 500 saturates to -448 -> 0xFE
    q, s = oracle.quant_mxfp8(blk)     # row 3 all zero -> byte 0, codes 0
    assert list(s[:, 0]) == [119, 127, 127, 0]
    assert q[0, 5] == 0x78 and q[0, 0] == 0
    assert np.all(q[1] == 0x7E)
    assert q[2, 3] == 0xFE
    assert np.all(q[3] == 0)


def test_mxfp8_rounding_error_bound():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))
    q, s = oracle.quant_mxfp8(v)
    d = oracle.dequant_mxfp8(q, s)
    scale = np.repeat(oracle.e8m0_decode(s), 32, axis=-1)
    scaled = np.abs(v) / scale
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448.0)
    # nearest rounding with a 3-bit mantissa: error at most 2^-4 of the value
    assert np.all(np.abs(d - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4)
    # subnormal elements: absolute error at most half a spacing (2^-10 * scale)
    sub = scaled < 2.0 ** -6
    assert np.all(np.abs(d - v)[sub] <= scale[sub] * 2.0 ** -10)


# ----------------------------------------------------------------- routing

def test_topk_selection_by_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(200):
        E, k = int(rng.integers(2, 9)), 0
        k = int(rng.integers(1, E + 1))
        lg = rng.integers(-3, 4, size=(1, E)).astype(np.float32)  # many ties
        ids, w = oracle.route_topk_softmax(lg, k)
        sel = list(ids[0])
        rest = [i for i in range(E) if i not in sel]
        l = lg[0]
        def before(a, b):  # a ranks before b: larger logit, or equal and lower id
            return l[a] > l[b] or (l[a] == l[b] and a < b)
        assert len(set(sel)) == k
        assert all(before(a, b) for a in sel for b in rest)
        assert all(before(sel[j], sel[j + 1]) for j in range(k - 1))


def test_topk_matches_torch_topk_on_distinct_logits():
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((50, 896)).astype(np.float32)
    ids, _ = oracle.route_topk_softmax(lg, 16)
    want = torch.topk(torch.from_numpy(lg), 16, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(ids, want)


def test_topk_weights_are_softmax_of_selected():
    rng = np.random.default_rng(13)
    lg = (rng.standard_normal((40, 64)) * 3).astype(np.float32)
    ids, w = oracle.route_topk_softmax(lg, 8)
    sel = np.take_along_axis(lg.astype(np.float64), ids, 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    renorm = np.take_along_axis(full, ids, 1)
    assert np.allclose(w, renorm / renorm.sum(1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_topk_non_finite_logits():
    """NaN ranks below -inf (ties by lower id) and a selected NaN has weight
    0; infinities follow IEEE arithmetic in exp(l - l_max)."""
    nan, inf = np.nan, np.inf
    lg = np.array([[1.0, nan, 0.5, -inf, 2.0],
                   [nan, nan, 1.0, nan, nan],
                   [-inf, 0.0, nan, -inf, nan],
                   [inf, 0.0, 1.0, nan, -1.0],
                   [nan, nan, nan, nan, nan],
                   [-inf, -inf, nan, 3.0, -inf]], np.float32)
    ids, w = oracle.route_topk_softmax(lg, 3)
    assert ids.tolist() == [[4, 0, 2], [2, 0, 1], [1, 0, 3], [0, 2, 1], [0, 1, 2], [3, 0, 1]]
    e = np.exp([0.0, -1.0, -1.5])
    assert np.allclose(w[0], e / e.sum(), rtol=1e-15, atol=0)
    assert w[1].tolist() == [1.0, 0.0, 0.0]
    assert w[2].tolist() == [1.0, 0.0, 0.0]
    assert np.all(np.isnan(w[3])) and np.all(np.isnan(w[4]))
    assert w[5].tolist() == [1.0, 0.0, 0.0]


def test_local_map_offset_and_masked_ids():
    ids = np.array([[-1, 0, 447, 448, 449, 895, 896, 1000]])
    got = oracle.local_map(ids, 448, 448)
    assert list(got[0]) == [-1, -1, -1, 0, 1, 447, -1, -1]


# ----------------------------------------------------------- shared append

def test_shared_append_golden_values():
    rows = _golden_rows("shared_append.txt")
    for lg, sc, want in rows:
        bits = f32_to_bf16_bits(np.array([[float(lg)]], np.float32))
        ids, w = oracle.shared_append(bits, E=10, S=1, scale=float(sc))
        assert ids[0, 0] == 10
        assert math.isclose(w[0, 0], float(want), rel_tol=1e-14, abs_tol=0)


def test_shared_append_matches_scipy_expit():
    rng = np.random.default_rng(5)
    bits = f32_to_bf16_bits((rng.standard_normal((64, 3)) * 2).astype(np.float32))
    ids, w = oracle.shared_append(bits, E=7, S=3, scale=0.5)
    assert np.array_equal(ids, np.broadcast_to([7, 8, 9], (64, 3)))
    want = scipy.special.expit(oracle.bf16_bits_to_f64(bits)) * 0.5
    assert np.allclose(w, want, rtol=1e-15, atol=0)


# -------------------------------------------------------------------- sort

def test_kmax_v_reproduces_kimi_k31_constant():
    g = {r[0]: int(r[1]) for r in _golden_rows("kimi_k31_tp8_shape.txt")}
    assert oracle.kmax_v(g["num_experts"], g["max_tokens"], g["top_k"], g["block_n"]) == g["kmax_v"]


def _check_sort(se, Ep, B):
    m = oracle.sort_align(se, Ep, B)
    flat = se.reshape(-1)
    # brute force: rows are the valid slots sorted by (expert, slot)
    want = [s for _, s in sorted((int(e), s) for s, e in enumerate(flat) if e >= 0)]
    assert list(m["sorted_slot"]) == want
    assert m["counts"].sum() == np.count_nonzero(flat >= 0)
    assert np.array_equal(m["counts"], np.bincount(flat[flat >= 0], minlength=Ep)[:Ep])
    assert m["offsets"][0] == 0 and np.all(np.diff(m["offsets"]) == m["counts"])
    R = len(want)
    ex = m["expanded_idx"]
    assert np.all(ex[flat < 0] == -1)
    assert np.array_equal(ex[m["sorted_slot"]], np.arange(R))
    # every row belongs to its expert's range
    for e in range(Ep):
        seg = m["sorted_slot"][m["offsets"][e]:m["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
    T, Kp = se.shape
    assert m["num_v"] <= oracle.kmax_v(Ep, T, Kp, B)
    # vinfo chunks tile each expert's rows in order
    covered = np.zeros(R, np.int64)
    for e, r0, n, c in m["vinfo"]:
        assert 1 <= n <= B and r0 == m["offsets"][e] + c * B
        covered[r0:r0 + n] += 1
        assert np.all(flat[m["sorted_slot"][r0:r0 + n]] == e)
    assert np.all(covered == 1)
    return m


def test_sort_brute_force_random():
    rng = np.random.default_rng(21)
    for _ in range(60):
        T, Kp, Ep = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 20))
        B = int(rng.choice([1, 2, 16, 32]))
        se = rng.integers(-1, Ep, size=(T, Kp)).astype(np.int32)
        _check_sort(se, Ep, B)


def test_sort_counts_sum_when_all_local():
    s = LayerShape("t", T=48, E=64, E_g=64, topk=16, H=512, I=128, B=16)
    inp = make_inputs(s, 9, weights=False)
    res = oracle.reference_forward(s, inp, compute_out=False)
    assert res["counts"].sum() == s.T * s.topk
    _check_sort(res["slot_expert"], s.Ep, s.B)


def test_vinfo_bound_is_tight():
    # every token on its own experts in chunks of exactly B reach the bound's shape
    T, Kp, B, Ep = 32, 2, 16, 8
    se = np.tile(np.arange(2, dtype=np.int32), (T, 1))  # two experts, 32 rows each
    m = _check_sort(se, Ep, B)
    assert m["num_v"] == 4


# -------------------------------------------------------------------- gate

def test_gate_rule_and_force():
    c = np.zeros(10, np.int32)
    assert oracle.gate_word(c) == (0, 0, 0, 0)
    c[:4] = [64, 64, 64, 63]
    assert oracle.gate_word(c)[:3] == (0, 4, 255)        # 255 < 64*4
    c[3] = 64
    assert oracle.gate_word(c) == (1, 4, 256, 4)
    c[0] = 129
    assert oracle.gate_word(c) == (1, 4, 321, 5)         # 129 rows -> two 128-row tiles
    assert oracle.gate_word(c, force_path=0) == (0, 4, 321, 0)
    c2 = np.array([1, 1, 0], np.int32)
    assert oracle.gate_word(c2, force_path=1) == (1, 2, 2, 2)
    t = oracle.dense_tiles(np.array([0, 300, 5]), np.array([0, 0, 300, 305]))
    assert t.tolist() == [[1, 0, 128, 0], [1, 128, 128, 1], [1, 256, 44, 2], [2, 300, 5, 0]]


# ------------------------------------------------- whole layer, closed form

def _pack_rows(codes):
    """codes [rows, K] (0..15) -> bytes [rows, K/2], low nibble = even k."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _onehot_layer(H=64, I=32, E=3, S=1):
    """A layer whose weights are one-hot rows, so its output has a closed form.

    Expert e: gate row i reads x[pg_e(i)] times cg_e, up row i reads
    x[pu_e(i)] times cu_e, output row h reads act[h % I] times c2_e.
    The other scale group of each row holds a different exponent, so a
    wrong group index changes the result.
    """
    Ep = E + S
    gcode, gscale = 3, 126   # 1.5 * 2^-1 = 0.75
    ucode, uscale = 6, 125   # 4.0 * 2^-2 = 1.0
    dcode, dscale = 5, 128   # 3.0 * 2^1 = 6.0
    w13c = np.zeros((Ep, 2 * I, H), np.uint8)
    s13 = np.zeros((Ep, 2 * I, H // 32), np.uint8)
    w2c = np.zeros((Ep, H, I), np.uint8)
    s2 = np.zeros((Ep, H, I // 32), np.uint8)
    pg = lambda e, i: (5 * i + 7 * e + 1) % H
    pu = lambda e, i: (3 * i + 11 * e + 2) % H
    for e in range(Ep):
        for i in range(I):
            k = pg(e, i)
            w13c[e, i, k] = gcode
            s13[e, i, :] = gscale + 3
            s13[e, i, k // 32] = gscale + e  # expert e's gate weight is 0.75 * 2^e
            k = pu(e, i)
            w13c[e, I + i, k] = ucode
            s13[e, I + i, :] = uscale + 2
            s13[e, I + i, k // 32] = uscale
        for h in range(H):
            w2c[e, h, h % I] = dcode
            s2[e, h, :] = dscale
    cgv = lambda e: 0.75 * 2.0 ** e
    wts = dict(w13=np.stack([_pack_rows(w13c[e]) for e in range(Ep)]), s13=s13,
               w2=np.stack([_pack_rows(w2c[e]) for e in range(Ep)]), s2=s2)
    return H, I, E, S, pg, pu, cgv, 1.0, 6.0, wts


def _closed_form_out(x, ids, w, shared_w, E, offset, limit, H, I, pg, pu, cgv, cu, c2,
                     act=("swiglu",)):
    silu = lambda v: v / (1.0 + math.exp(-v))
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    T = x.shape[0]
    out = np.zeros((T, H))
    for t in range(T):
        cols = [(int(g) - offset, float(wt)) for g, wt in zip(ids[t], w[t])
                if g >= 0 and 0 <= int(g) - offset < E]
        cols += [(E + s, float(shared_w[t, s])) for s in range(shared_w.shape[1])]
        for e, wt in cols:
            for h in range(H):
                i = h % I
                g = cgv(e) * x[t, pg(e, i)]
                u = cu * x[t, pu(e, i)]
                if act[0] == "situ":
                    beta, lb = act[1], act[2]
                    out[t, h] += wt * c2 * (beta * math.tanh(g / beta) * sig(g)) * (lb * math.tanh(u / lb))
                    continue
                if limit > 0:
                    g = min(g, limit)
                    u = max(-limit, min(u, limit))
                out[t, h] += wt * c2 * silu(g) * u
    return out


@pytest.mark.parametrize("limit", [0.0, 1.25])
def test_whole_layer_closed_form(limit, act=("swiglu",)):
    H, I, E, S, pg, pu, cgv, cu, c2, wts = _onehot_layer()
    offset, E_g, topk, T = 2, 8, 3, 5
    rng = np.random.default_rng(31)
    x = (rng.integers(-16, 17, size=(T, H)) / 4.0).astype(np.float32)  # exact in bf16
    ids = np.array([[2, 3, 4], [0, 3, -1], [5, 7, 1], [4, 2, 6], [-1, -1, -1]], np.int32)
    w = np.array([[.5, .25, .25], [.3, .7, 0], [.6, .3, .1], [.125, .5, .375], [1, 0, 0]], np.float32)
    sh = f32_to_bf16_bits(np.array([[0.0], [2.0], [-2.0], [1.0], [0.5]], np.float32))
    shape = LayerShape("cf", T=T, E=E, E_g=E_g, topk=topk, H=H, I=I, B=2, S=S,
                       expert_offset=offset, swiglu_limit=limit, shared_scale=0.5, mode="ids")
    if act[0] == "situ":
        shape = shape.replace(activation="situ", act_beta=act[1], act_linear_beta=act[2])
    inp = dict(x=f32_to_bf16_bits(x), logits=np.zeros((T, E_g), np.float32), shared=sh,
               topk_ids=ids, topk_w=w, **wts)
    got = oracle.reference_forward(shape, inp)["out"]
    shared_w = scipy.special.expit(oracle.bf16_bits_to_f64(sh)) * 0.5
    want = _closed_form_out(x.astype(np.float64), ids, w.astype(np.float64), shared_w, E, offset,
                            limit, H, I, pg, pu, cgv, cu, c2, act)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    if limit > 0:  # the clamp must actually bite in this example
        g_all = [cgv(e) * abs(x[t, pg(e, i)]) for t in range(T) for e in range(E + S) for i in range(I)]
        assert max(g_all) > limit


# ------------------------------------------------------------------ SiTU
# [SHAPE] section 4 prints the SiTU activation of the K3.1 kernel for
# beta = 4 and linear beta = 25 only: gate factor 2 tanh(g/4)(1 + tanh(g/2)),
# up factor 25 tanh(u/25). The oracle's general form beta tanh(g/beta)
# sigmoid(g) * lb tanh(u/lb) must reproduce that instance, and must reduce
# to SwiGLU when both caps go to infinity.

def test_situ_matches_printed_instance():
    g, u = np.meshgrid(np.linspace(-60, 60, 241), np.linspace(-80, 80, 161))
    printed = (2.0 * np.tanh(g * 0.25) * (1.0 + np.tanh(g * 0.5))) * (25.0 * np.tanh(u * 0.04))
    got = oracle.situ(g, u, 4.0, 25.0)
    assert np.max(np.abs(got - printed)) <= 1e-12 * np.max(np.abs(printed))


def test_situ_reduces_to_swiglu_without_caps():
    rng = np.random.default_rng(5)
    g, u = rng.normal(0, 5, 1000), rng.normal(0, 5, 1000)
    swiglu = g * scipy.special.expit(g) * u
    got = oracle.situ(g, u, 1e9, 1e9)
    assert np.allclose(got, swiglu, rtol=1e-9, atol=1e-12)


def test_situ_caps_symmetry_and_zero():
    beta, lb = 4.0, 25.0
    g = np.linspace(-50, 50, 1001)
    one = np.ones_like(g)
    # odd in u, zero at g = 0, bounded by beta * lb
    assert np.allclose(oracle.situ(g, -3 * one, beta, lb), -oracle.situ(g, 3 * one, beta, lb))
    assert oracle.situ(np.zeros(1), np.ones(1), beta, lb)[0] == 0.0
    assert np.all(np.abs(oracle.situ(g, 1e6 * one, beta, lb)) <= beta * lb * (1 + 1e-12))
    # the gate factor tends to beta for large g and to 0 for very negative g
    big = oracle.situ(np.array([200.0]), np.array([lb * np.arctanh(0.5)]), beta, lb)[0]
    assert abs(big - beta * 0.5 * lb) <= 1e-9
    assert abs(oracle.situ(np.array([-200.0]), np.array([1.0]), beta, lb)[0]) < 1e-60


@pytest.mark.parametrize("beta,lb", [(4.0, 25.0), (1.5, 0.75)])
def test_whole_layer_closed_form_situ(beta, lb):
    test_whole_layer_closed_form(0.0, ("situ", beta, lb))


def test_dense_glu_reduction_matches_torch():
    # E = 1, top-1, weight 1: the layer is a plain gated MLP,
    # y = W2 (silu(Wg x) * (Wu x)), evaluated with torch in float64.
    s = LayerShape("glu", T=6, E=1, E_g=1, topk=1, H=64, I=32, B=16, exp_lo=120, exp_hi=127)
    inp = make_inputs(s, 17)
    got = oracle.reference_forward(s, inp)["out"]
    table = torch.from_numpy(_e2m1_table())

    def deq(packed, sc):
        p = torch.from_numpy(packed.astype(np.int64))
        codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1)
        scale = torch.from_numpy(sc).view(torch.float8_e8m0fnu).double()
        return table[codes] * scale.repeat_interleave(32, dim=1)

    W13 = deq(inp["w13"][0], inp["s13"][0])
    W2 = deq(inp["w2"][0], inp["s2"][0])
    x = torch.from_numpy(inp["x"].astype(np.int32)).to(torch.int16).view(torch.bfloat16).double()
    Wg, Wu = W13[:32], W13[32:]
    y = torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T) @ W2.T
    assert np.allclose(got, y.numpy(), rtol=1e-12, atol=1e-9)


# ------------------------------------------------ grouped vs per-token loop

SMALL = [
    LayerShape("s1", T=9, E=8, E_g=8, topk=2, H=64, I=32, B=2),
    LayerShape("s2", T=17, E=6, E_g=12, topk=4, H=64, I=64, B=3, expert_offset=6, routing="zipf"),
    LayerShape("s3", T=11, E=5, E_g=5, topk=2, H=96, I=32, B=4, S=2, swiglu_limit=3.0,
               shared_scale=0.5),
    LayerShape("s4", T=13, E=7, E_g=20, topk=5, H=64, I=32, B=2, expert_offset=3, mode="ids"),
    LayerShape("s5", T=7, E=4, E_g=4, topk=2, H=64, I=64, B=16, a_dtype="mxfp8", S=1,
               swiglu_limit=2.0),
    LayerShape("s6_situ", T=10, E=6, E_g=6, topk=3, H=64, I=32, B=2, S=1, activation="situ"),
    LayerShape("s7_a4", T=9, E=5, E_g=5, topk=2, H=64, I=64, B=2, S=1, swiglu_limit=3.0,
               a_dtype="mxfp4"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: s.name)
def test_grouped_matches_per_token_loop(shape):
    inp = make_inputs(shape, 100 + SMALL.index(shape))
    if shape.mode == "ids":
        inp["topk_ids"][0, 0] = -1
        inp["topk_ids"][1, :] = -1
    res = oracle.reference_forward(shape, inp)
    loop = oracle.sampled_forward(shape, inp, np.arange(shape.T))
    assert np.allclose(res["out"], loop, rtol=1e-12, atol=1e-9 * np.max(np.abs(loop)))
    sub = np.array([shape.T - 1, 0, 2])
    assert np.allclose(oracle.sampled_forward(shape, inp, sub), res["out"][sub],
                       rtol=1e-12, atol=1e-9 * np.max(np.abs(loop)))


def test_finalize_zero_and_single_slot():
    s = LayerShape("z", T=4, E=4, E_g=8, topk=1, H=64, I=32, B=2, expert_offset=4, mode="ids")
    inp = make_inputs(s, 41)
    inp["topk_ids"][:] = np.array([[0], [3], [5], [-1]])
    inp["topk_w"][:] = np.array([[1.0], [0.5], [0.25], [1.0]], np.float32)
    res = oracle.reference_forward(s, inp)
    out = res["out"]
    assert np.all(out[0] == 0) and np.all(out[1] == 0) and np.all(out[3] == 0)
    x = oracle.bf16_bits_to_f64(inp["x"][2:3])
    W13 = oracle.dequant_mxfp4(inp["w13"][1], inp["s13"][1])
    W2 = oracle.dequant_mxfp4(inp["w2"][1], inp["s2"][1])
    assert np.allclose(out[2], 0.25 * oracle.expert_glu(x, W13, W2)[0], rtol=1e-14, atol=0)


def test_mxfp8_activation_path_quantises_x_per_token():
    s = SMALL[4]
    inp = make_inputs(s, 104)
    res = oracle.reference_forward(s, inp, compute_out=False)
    q, sc = oracle.quant_mxfp8(oracle.bf16_bits_to_f64(inp["x"]))
    assert np.array_equal(res["xq"], q) and np.array_equal(res["xs"], sc)
    assert res["xq"].shape == (s.T, s.H) and res["xs"].shape == (s.T, s.H // 32)


# ------------------------------------- W4A8: where MXFP8 enters the layer
# The W4A8 layer quantises x to MXFP8 per 32 elements along H before GEMM1,
# and the activation output act per 32 elements along I after the activation
# and before GEMM2 (the Shape-template page, section 7, names MXFP8
# activations for the decode MoE; the recipe is OCP MX). This pin computes
# that composition by hand on a one-hot layer: block scales from math.frexp,
# element rounding by torch's float8_e4m3fn cast, and the activation from
# math.exp, sharing nothing with the oracle's quantiser.

def _e4m3_midpoint(v32: np.ndarray) -> np.ndarray:
    """True where a float32 value lies exactly halfway between two E4M3
    values (where rounding float64 -> float32 -> E4M3 could differ from a
    direct rounding)."""
    a = np.abs(v32.astype(np.float64))
    m, e = np.frexp(a)
    normal = a >= 2.0 ** -6
    mid_n = (np.floor(m * 32) == m * 32) & (np.floor(m * 16) != m * 16)
    k = a * 2.0 ** 10
    mid_s = (np.floor(k) == k) & (np.mod(k, 2) == 1)
    return np.where(normal, mid_n, mid_s) & (a <= 448.0)


def _mxfp8_by_hand(v: np.ndarray) -> np.ndarray:
    """MXFP8 round trip along the last axis, blocks of 32: shared exponent
    floor(log2 amax) - 8 (biased, clamped to [0, 254]), elements rounded to
    E4M3 by torch with saturation at 448."""
    v = np.asarray(v, np.float64)
    out = np.zeros_like(v)
    for idx in np.ndindex(v.shape[:-1]):
        for b in range(v.shape[-1] // 32):
            blk = v[idx][32 * b: 32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            if amax == 0.0:
                continue
            _, e = math.frexp(amax)  # amax = m 2^e, m in [0.5, 1)
            se = min(max(e - 1 - 8 + 127, 0), 254) - 127
            scaled = np.clip(blk / 2.0 ** se, -448.0, 448.0)
            s32 = scaled.astype(np.float32)
            assert not np.any(_e4m3_midpoint(s32) & (s32.astype(np.float64) != scaled))
            q = torch.from_numpy(s32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            out[idx][32 * b: 32 * b + 32] = q * 2.0 ** se
    return out


def _w4a8_onehot_case():
    """32 tokens, every one routed to both local experts plus one shared
    expert, so each expert holds 32 rows (a wrong quantisation axis over
    rows is computable and must fail). H = I = 64: two MX blocks along each."""
    H, I, E, S = 64, 64, 2, 1
    _, _, _, _, pg, pu, cgv, cu, c2, wts = _onehot_layer(H, I, E, S)
    T = 32
    rng = np.random.default_rng(47)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * np.float32(1.7))
    xf = oracle.bf16_bits_to_f64(x)
    # a saturating block: amax 480 scales to 480 > 448 and saturates
    x[3, 0:32] = f32_to_bf16_bits(np.linspace(-2.0, 2.0, 32).astype(np.float32))
    x[3, 7] = f32_to_bf16_bits(np.array([480.0], np.float32))[0]
    # an underflowing block: elements far below amax / 2^8 round to zero
    x[5, 32:64] = f32_to_bf16_bits((np.arange(32) % 7 - 3).astype(np.float32) * np.float32(2 ** -20))
    x[5, 40] = f32_to_bf16_bits(np.array([3.0], np.float32))[0]
    xf = oracle.bf16_bits_to_f64(x)
    ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    w = (rng.random((T, 2)) + 0.1).astype(np.float32)
    sh = f32_to_bf16_bits((rng.standard_normal((T, 1)) * 2).astype(np.float32))
    shape = LayerShape("cf_a8", T=T, E=E, E_g=E, topk=2, H=H, I=I, B=16, S=S, shared_scale=1.0,
                       a_dtype="mxfp8", mode="ids")
    inp = dict(x=x, logits=np.zeros((T, E), np.float32), shared=sh, topk_ids=ids, topk_w=w, **wts)
    # the closed form, by hand
    xd = _mxfp8_by_hand(xf)
    assert np.any(xd != xf)                          # x quantisation changes x
    assert xd[3, 7] == 448.0                         # saturated
    assert np.all(xd[5, 32:64][np.arange(32) != 8] == 0.0) and xd[5, 40] == 3.0  # underflowed
    shared_w = scipy.special.expit(oracle.bf16_bits_to_f64(sh))[:, 0]
    out = np.zeros((T, H))
    for e, wt in ((0, w[:, 0].astype(np.float64)), (1, w[:, 1].astype(np.float64)), (2, shared_w)):
        act = np.zeros((T, I))
        for t in range(T):
            for i in range(I):
                g = cgv(e) * xd[t, pg(e, i)]
                u = cu * xd[t, pu(e, i)]
                act[t, i] = g / (1.0 + math.exp(-g)) * u
        actq = _mxfp8_by_hand(act)
        assert np.any(actq != act)
        out += wt[:, None] * c2 * actq[:, np.arange(H) % I]
    return shape, inp, out


def test_w4a8_composition_closed_form():
    shape, inp, want = _w4a8_onehot_case()
    got = oracle.reference_forward(shape, inp)["out"]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def _w4a8_closed_form_error():
    try:
        test_w4a8_composition_closed_form()
    except AssertionError:
        return True
    return False


def test_w4a8_planted_mistakes_are_caught(monkeypatch):
    assert not _w4a8_closed_form_error()
    orig_glu, orig_act = omoe.expert_glu, omoe._activations
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    rt = lambda v: omx.dequant_mxfp8(*omx.quant_mxfp8(v))
    # 1. act not quantised before GEMM2
    monkeypatch.setattr(omoe, "expert_glu",
                        lambda xr, W13, W2, limit=0.0, act_quant="bf16", **kw:
                        orig_glu(xr, W13, W2, limit, "bf16", **kw))
    assert _w4a8_closed_form_error()

    # 2. the GEMM1 outputs g and u quantised before the activation instead of act
    def glu_h_quant(xr, W13, W2, limit=0.0, act_quant="bf16", **kw):
        I = W13.shape[0] // 2
        h = xr @ W13.T
        g, u = rt(h[:, :I]), rt(h[:, I:])
        return (g * sig(g) * u) @ W2.T
    monkeypatch.setattr(omoe, "expert_glu", glu_h_quant)
    assert _w4a8_closed_form_error()

    # 3. act quantised along the rows (tokens) instead of along I
    def glu_act_along_t(xr, W13, W2, limit=0.0, act_quant="bf16", **kw):
        I = W13.shape[0] // 2
        h = xr @ W13.T
        g, u = h[:, :I], h[:, I:]
        return rt((g * sig(g) * u).T).T @ W2.T
    monkeypatch.setattr(omoe, "expert_glu", glu_act_along_t)
    assert _w4a8_closed_form_error()
    monkeypatch.setattr(omoe, "expert_glu", orig_glu)

    # 4. x quantised along T instead of along H
    def act_x_along_t(shape, inp):
        x = omoe.bf16_bits_to_f64(inp["x"])
        return rt(x.T).T, None, None
    monkeypatch.setattr(omoe, "_activations", act_x_along_t)
    assert _w4a8_closed_form_error()

    # 5. x not quantised
    monkeypatch.setattr(omoe, "_activations",
                        lambda shape, inp: (omoe.bf16_bits_to_f64(inp["x"]), None, None))
    assert _w4a8_closed_form_error()
    monkeypatch.setattr(omoe, "_activations", orig_act)
    assert not _w4a8_closed_form_error()


# -------------------------------------------------- MXFP4 (W4A4) activations
# "SGLang CUTLASS MoE", section 6: FP4 (E2M1) activations as well as
# weights. Here in the weights' own MX block format: one E8M0 per 32, shared
# exponent floor(log2 amax) - 2, nearest E2M1 value with ties to the even
# code, saturation at 6.

def _e2m1_nearest_by_hand(m: float) -> int:
    """Brute force over the eight magnitudes of the golden table: the nearest,
    a tie to the even code; m >= 0."""
    table = _e2m1_table()[:8]
    m = min(m, 6.0)
    best = None
    for code in range(8):
        d = abs(m - table[code])
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def test_e2m1_encode_by_brute_force():
    rng = np.random.default_rng(17)
    table = _e2m1_table()[:8]
    mids = (table[1:] + table[:-1]) / 2
    v = np.concatenate([rng.uniform(-7.5, 7.5, 4000), rng.uniform(-0.6, 0.6, 1000), table, mids,
                        [6.0, 6.5, 7.0, 100.0, 1e-30]])
    v = np.concatenate([v, -v])
    got = omx._e2m1_encode(v)
    want = [_e2m1_nearest_by_hand(abs(x)) | (8 if x < 0 or (x == 0 and math.copysign(1, x) < 0) else 0)
            for x in v]
    assert list(got) == want
    # ties between neighbours go to the even code: 0.25 -> 0, 0.75 -> 1.0,
    # 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0
    assert list(omx._e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]


def test_mxfp4_shared_exponent_worked_examples():
    blk = np.zeros((5, 32))
    blk[0, 5] = 1.0      # amax 1 -> exponent -2 -> byte 125; 1.0 / 0.25 = 4 -> code 6
    blk[1, :] = 6.0      # amax 6 -> exponent 0 -> byte 127; 6 -> code 7
    blk[2, 3] = -7.0     # amax 7 -> exponent 0; -7 saturates to -6 -> code 15
    blk[2, 4] = 0.2      # 0.2 -> 0 (nearest)
    blk[4, 0] = -0.001   # rounds to -0 under amax 3: code 8
    blk[4, 1] = 3.0      # amax 3 -> exponent -1 -> byte 126; 3 / 0.5 = 6 -> code 7
    q, s = oracle.quant_mxfp4(blk)        # row 3 all zero -> byte 0, codes 0
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(5, 32)
    assert list(s[:, 0]) == [125, 127, 127, 0, 126]
    assert codes[0, 5] == 6 and np.count_nonzero(codes[0]) == 1
    assert np.all(codes[1] == 7)
    assert codes[2, 3] == 15 and codes[2, 4] == 0
    assert np.all(codes[3] == 0)
    assert codes[4, 0] == 8 and codes[4, 1] == 7
    d = oracle.dequant_mxfp4(q, s)
    assert d[0, 5] == 1.0 and d[2, 3] == -6.0 and d[4, 1] == 3.0


def test_mxfp4_rounding_error_bound():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))
    q, s = oracle.quant_mxfp4(v)
    d = oracle.dequant_mxfp4(q, s)
    scale = np.repeat(oracle.e8m0_decode(s), 32, axis=-1)
    m = np.abs(v) / scale
    # spacing of E2M1 values at magnitude m: 0.5 below 2, 1 below 4, 2 above
    half = np.where(m < 2, 0.25, np.where(m < 4, 0.5, 1.0)) * scale
    inside = m <= 6.0
    assert np.all(np.abs(d - v)[inside] <= half[inside])
    assert np.all(np.abs(d[~inside]) == 6.0 * scale[~inside])  # saturated
    assert np.all(m < 8.0)  # the shared exponent keeps every block below 2^3


def _mxfp4_by_hand(v: np.ndarray) -> np.ndarray:
    """MXFP4 round trip along the last axis, blocks of 32, by plain loops."""
    table = _e2m1_table()[:8]
    v = np.asarray(v, np.float64)
    out = np.zeros_like(v)
    for idx in np.ndindex(v.shape[:-1]):
        for b in range(v.shape[-1] // 32):
            blk = v[idx][32 * b: 32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            if amax == 0.0:
                continue
            _, e = math.frexp(amax)
            se = min(max(e - 1 - 2 + 127, 0), 254) - 127
            for j, x in enumerate(blk):
                code = _e2m1_nearest_by_hand(abs(x) / 2.0 ** se)
                out[idx][32 * b + j] = math.copysign(table[code] * 2.0 ** se, x)
    return out


def _w4a4_onehot_case():
    """The W4A8 one-hot case with MXFP4 activations (x along H, act along I)."""
    H, I, E, S = 64, 64, 2, 1
    _, _, _, _, pg, pu, cgv, cu, c2, wts = _onehot_layer(H, I, E, S)
    T = 32
    rng = np.random.default_rng(53)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * np.float32(1.7))
    x[3, 0:32] = f32_to_bf16_bits(np.linspace(-2.0, 2.0, 32).astype(np.float32))
    x[3, 7] = f32_to_bf16_bits(np.array([14.0], np.float32))[0]   # 14 / 2 = 7 saturates to 6
    x[5, 32:64] = f32_to_bf16_bits((np.arange(32) % 7 - 3).astype(np.float32) * np.float32(2 ** -6))
    x[5, 40] = f32_to_bf16_bits(np.array([3.0], np.float32))[0]  # the others round to zero
    # a block of exact E2M1 midpoints (amax 5 -> shared exponent 0): each a tie
    x[7, 0:32] = f32_to_bf16_bits(np.resize(np.array(
        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0],
        np.float32), 32))
    xf = oracle.bf16_bits_to_f64(x)
    ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    w = (rng.random((T, 2)) + 0.1).astype(np.float32)
    sh = f32_to_bf16_bits((rng.standard_normal((T, 1)) * 2).astype(np.float32))
    shape = LayerShape("cf_a4", T=T, E=E, E_g=E, topk=2, H=H, I=I, B=16, S=S, shared_scale=1.0,
                       a_dtype="mxfp4", mode="ids")
    inp = dict(x=x, logits=np.zeros((T, E), np.float32), shared=sh, topk_ids=ids, topk_w=w, **wts)
    xd = _mxfp4_by_hand(xf)
    assert np.any(xd != xf)
    assert xd[3, 7] == 12.0                           # saturated: 6 * 2^1
    assert np.all(xd[5, 32:64][np.arange(32) != 8] == 0.0) and xd[5, 40] == 3.0
    assert list(xd[7, 0:7]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]  # ties to the even code
    shared_w = scipy.special.expit(oracle.bf16_bits_to_f64(sh))[:, 0]
    out = np.zeros((T, H))
    for e, wt in ((0, w[:, 0].astype(np.float64)), (1, w[:, 1].astype(np.float64)), (2, shared_w)):
        act = np.zeros((T, I))
        for t in range(T):
            for i in range(I):
                g = cgv(e) * xd[t, pg(e, i)]
                u = cu * xd[t, pu(e, i)]
                act[t, i] = g / (1.0 + math.exp(-g)) * u
        actq = _mxfp4_by_hand(act)
        assert np.any(actq != act)
        out += wt[:, None] * c2 * actq[:, np.arange(H) % I]
    return shape, inp, out


def test_w4a4_composition_closed_form():
    shape, inp, want = _w4a4_onehot_case()
    res = oracle.reference_forward(shape, inp)
    assert np.max(np.abs(res["out"] - want)) <= 1e-12 * np.max(np.abs(want))
    assert res["xq"].shape == (shape.T, shape.H // 2) and res["xs"].shape == (shape.T, shape.H // 32)


def _w4a4_closed_form_error():
    try:
        test_w4a4_composition_closed_form()
    except AssertionError:
        return True
    return False


def test_w4a4_planted_mistakes_are_caught(monkeypatch):
    assert not _w4a4_closed_form_error()
    orig_glu, orig_act = omoe.expert_glu, omoe._activations
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    rt4 = lambda v: omx.dequant_mxfp4(*omx.quant_mxfp4(v))
    rt8 = lambda v: omx.dequant_mxfp8(*omx.quant_mxfp8(v))
    # 1. act not quantised; 2. act quantised to MXFP8 instead of MXFP4
    for fmt in ("bf16", "mxfp8"):
        monkeypatch.setattr(omoe, "expert_glu",
                            lambda xr, W13, W2, limit=0.0, act_quant="bf16", fmt=fmt, **kw:
                            orig_glu(xr, W13, W2, limit, fmt, **kw))
        assert _w4a4_closed_form_error(), fmt

    # 3. g and u quantised before the activation instead of act
    def glu_h_quant(xr, W13, W2, limit=0.0, act_quant="bf16", **kw):
        I = W13.shape[0] // 2
        h = xr @ W13.T
        g, u = rt4(h[:, :I]), rt4(h[:, I:])
        return (g * sig(g) * u) @ W2.T
    monkeypatch.setattr(omoe, "expert_glu", glu_h_quant)
    assert _w4a4_closed_form_error()

    # 4. act quantised along the rows
    def glu_act_along_t(xr, W13, W2, limit=0.0, act_quant="bf16", **kw):
        I = W13.shape[0] // 2
        h = xr @ W13.T
        g, u = h[:, :I], h[:, I:]
        return rt4((g * sig(g) * u).T).T @ W2.T
    monkeypatch.setattr(omoe, "expert_glu", glu_act_along_t)
    assert _w4a4_closed_form_error()
    monkeypatch.setattr(omoe, "expert_glu", orig_glu)

    # 5. x quantised along T; 6. x not quantised; 7. x quantised to MXFP8
    for fn in (lambda x: rt4(x.T).T, lambda x: x, rt8):
        monkeypatch.setattr(omoe, "_activations",
                            lambda shape, inp, fn=fn: (fn(omoe.bf16_bits_to_f64(inp["x"])),
                                                       np.zeros((shape.T, shape.H // 2), np.uint8),
                                                       np.zeros((shape.T, shape.H // 32), np.uint8)))
        assert _w4a4_closed_form_error()
    monkeypatch.setattr(omoe, "_activations", orig_act)

    # 8. ties rounded away from zero instead of to the even code
    orig_enc = omx._e2m1_encode

    def enc_ties_away(a):
        a = np.asarray(a, np.float64)
        return orig_enc(np.where(a == 0, a, a * (1 + 1e-12)))
    monkeypatch.setattr(omx, "_e2m1_encode", enc_ties_away)
    assert _w4a4_closed_form_error()
    monkeypatch.setattr(omx, "_e2m1_encode", orig_enc)
    assert not _w4a4_closed_form_error()


# ----------------------------------------------- planted mistakes are caught

def _closed_form_error(limit=1.25):
    try:
        test_whole_layer_closed_form(limit)
    except AssertionError:
        return True
    return False


def _situ_closed_form_error():
    try:
        test_whole_layer_closed_form_situ(1.5, 0.75)
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    assert not _closed_form_error()
    # 1. swapped nibble order
    orig_unpack = omx._unpack_nibbles

    def swapped(p):
        c = orig_unpack(p)
        return c.reshape(c.shape[:-1] + (-1, 2))[..., ::-1].reshape(c.shape)
    monkeypatch.setattr(omx, "_unpack_nibbles", swapped)
    assert _closed_form_error()
    monkeypatch.setattr(omx, "_unpack_nibbles", orig_unpack)
    # 2. gate and up halves swapped
    orig_glu = omoe.expert_glu

    def glu_swapped(xr, W13, W2, limit=0.0, act_quant="bf16", **act):
        I = W13.shape[0] // 2
        return orig_glu(xr, np.concatenate([W13[I:], W13[:I]]), W2, limit, act_quant, **act)
    monkeypatch.setattr(omoe, "expert_glu", glu_swapped)
    assert _closed_form_error()
    monkeypatch.setattr(omoe, "expert_glu", orig_glu)
    # 3. scale group index taken modulo instead of divided
    orig_deq = omoe.dequant_mxfp4

    def deq_bad(packed, scales):
        codes = omx._unpack_nibbles(packed)
        k = codes.shape[-1]
        idx = np.arange(k) % scales.shape[-1]
        return omx.e2m1_decode(codes) * omx.e8m0_decode(scales)[..., idx]
    monkeypatch.setattr(omoe, "dequant_mxfp4", deq_bad)
    assert _closed_form_error()
    monkeypatch.setattr(omoe, "dequant_mxfp4", orig_deq)
    # 4. gate clamped from below as well as above
    def glu_clamp_both(xr, W13, W2, limit=0.0, act_quant="bf16", **act):
        I = W13.shape[0] // 2
        h = xr @ W13.T
        g, u = h[:, :I], h[:, I:]
        if limit > 0:
            g, u = np.clip(g, -limit, limit), np.clip(u, -limit, limit)
        return (g / (1 + np.exp(-g)) * u) @ W2.T
    monkeypatch.setattr(omoe, "expert_glu", glu_clamp_both)
    assert _closed_form_error()
    monkeypatch.setattr(omoe, "expert_glu", orig_glu)
    # 5. expert offset ignored
    orig_lm = omoe.local_map
    monkeypatch.setattr(omoe, "local_map", lambda ids, E, off: orig_lm(ids, E, 0))
    assert _closed_form_error()
    monkeypatch.setattr(omoe, "local_map", orig_lm)
    # 7. SiTU caps swapped (beta on the up half, linear beta on the gate)
    orig_situ = omoe.situ
    monkeypatch.setattr(omoe, "situ", lambda g, u, b, lb: orig_situ(g, u, lb, b))
    assert _situ_closed_form_error()
    monkeypatch.setattr(omoe, "situ", orig_situ)
    assert not _situ_closed_form_error()
    # 6. shared weight without the sigmoid
    orig_sig = omoe._sigmoid
    monkeypatch.setattr(omoe, "shared_append",
                        lambda b, E, S, sc: (np.broadcast_to(np.arange(E, E + S, dtype=np.int32),
                                                             (b.shape[0], S)).copy(),
                                             omoe.bf16_bits_to_f64(b).reshape(-1, S) * sc))
    assert _closed_form_error()
    assert orig_sig is omoe._sigmoid
