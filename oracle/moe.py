"""The fused MXFP4 MoE expert layer, step by step, in float64.

Test infrastructure (see the package docstring). Each function follows one
passage of the sources, cited by page title and section:

  [CUTLASS]  "SGLang CUTLASS MoE: expert compute on optimised GEMM kernels"
  [SHAPE]    "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape
             template" (sglang PR 49091)
  [SHARED]   "SGLang MoE shared-expert optimisation: fusing three kernels
             into one" (sglang PR 28658)
  [GATE]     "Device-side gating of the MoE GEMM2 path" (flashinfer PR 6411)
  [MARLIN]   "MXFP4 Marlin MoE kernel for DeepSeek-V4" (sglang PR 24490)
"""
from __future__ import annotations

import numpy as np

from .mx import dequant_mxfp4, dequant_mxfp8, quant_mxfp4, quant_mxfp8

# Activation formats of the layer: the A operand of both GEMMs. "bf16" is
# W4A16; "mxfp8" (W4A8) and "mxfp4" (W4A4) quantise x along H before GEMM1
# and act along I before GEMM2.
_ACT_QUANT = {"mxfp8": (quant_mxfp8, dequant_mxfp8), "mxfp4": (quant_mxfp4, dequant_mxfp4)}

# Device GEMM2 gate: the dense path is taken when the routed rows average at
# least GATE_TAU per touched expert ([GATE] names the Dense and Split paths
# but not the rule; this threshold is this implementation's reading).
GATE_TAU = 64
# Row tile of the dense GEMM2 path's per-expert tile list.
DENSE_MT = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def route_topk_softmax(logits: np.ndarray, topk: int):
    """Softmax top-k routing with renormalisation over the selected experts.

    Per token the topk largest logits are taken in descending order; equal
    logits go to the lower expert id (a stable sort of -logit). The weights
    are the softmax of the selected logits, which equals the full softmax
    renormalised over the top-k. The pages consume the result of this step
    (the [T, top-k] ids the routing kernel reads, [SHAPE] section 5; the
    StandardTopKOutput of [SHARED]) without defining it; the configs ask for
    "softmax top-k renormalised".
    Non-finite logits (the pages do not treat them; this is the reading):
    a NaN logit ranks below every number, -inf included, NaNs among
    themselves by lower id, so it is selected only when fewer than topk
    logits are numbers; a selected NaN takes no part in the softmax
    (weight 0). Infinities follow IEEE arithmetic: exp(l - l_max) with
    l_max = +inf, or with every selected logit -inf, is NaN, and so are
    then all of the token's weights.
    Returns ids int32 [T, topk] (global expert ids) and w float64 [T, topk].
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    # argsort places NaN after every number, in index order (stable)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(lg, order, axis=1)
    with np.errstate(invalid="ignore"):
        ex = np.where(np.isnan(sel), 0.0, np.exp(sel - sel[:, :1]))
        return order.astype(np.int32), ex / ex.sum(axis=1, keepdims=True)


def local_map(ids: np.ndarray, E: int, expert_offset: int) -> np.ndarray:
    """Global expert ids -> local expert index, or -1.

    [SHAPE] section 5: an id outside [expert_offset, expert_offset + E), and
    the masked id -1, get no row; their expanded index is -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    loc = ids - expert_offset
    ok = (ids >= 0) & (loc >= 0) & (loc < E)
    return np.where(ok, loc, -1).astype(np.int32)


def shared_append(shared_bits: np.ndarray, E: int, S: int, scale: float):
    """The appended shared-expert columns.

    [SHARED], the append kernel after the change: shared column s of a token
    gets expert N_BASE + s and weight sigmoid(float32(bf16 logit)) * scale.
    Here N_BASE is the local expert count E (the shared experts' weights sit
    after the routed local experts), and the sigmoid is exact.
    Returns experts int32 [T, S] and weights float64 [T, S].
    """
    T = shared_bits.shape[0]
    lg = bf16_bits_to_f64(shared_bits).reshape(T, S)
    ids = np.broadcast_to(np.arange(E, E + S, dtype=np.int32), (T, S)).copy()
    return ids, _sigmoid(lg) * float(scale)


def kmax_v(Ep: int, T: int, Kp: int, B: int) -> int:
    """Upper bound on virtual experts (per-expert chunks of at most B rows).

    [SHAPE] section 1: the sum over touched experts of ceil(n_e / BlockN) is
    at most E + T*top-k/BlockN; with the shared columns the row count is
    T*K' and the expert count E' = E + S.
    """
    return Ep + (T * Kp) // B


def sort_align(slot_expert: np.ndarray, Ep: int, B: int) -> dict:
    """Group the token slots by expert into contiguous rows and B-row chunks.

    The slot of (token t, column k) is t*K' + k. [CUTLASS] section 1 builds
    per-expert offsets and the permutation (a_map) and its inverse (c_map);
    [SHAPE] section 5 keeps slots of one expert in token order (bitmask +
    popcount ranking) and marks slots without a local expert with -1.
    Rows of one expert are in ascending slot order.

    Returns counts [Ep], offsets [Ep+1], sorted_slot [R] (row -> slot),
    expanded_idx [T*K'] (slot -> row or -1), vinfo [num_v, 4] with rows
    (expert, first_row, rows, chunk) in expert-major then chunk order.
    """
    flat = np.asarray(slot_expert, dtype=np.int64).reshape(-1)
    slots = np.nonzero(flat >= 0)[0]
    ex = flat[slots]
    order = np.argsort(ex, kind="stable")
    sorted_slot = slots[order].astype(np.int32)
    counts = np.bincount(ex, minlength=Ep).astype(np.int32)[:Ep]
    offsets = np.zeros(Ep + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    expanded = np.full(flat.shape[0], -1, dtype=np.int32)
    expanded[sorted_slot] = np.arange(sorted_slot.shape[0], dtype=np.int32)
    vinfo = []
    for e in np.nonzero(counts)[0]:
        n = int(counts[e])
        for c in range((n + B - 1) // B):
            vinfo.append((int(e), int(offsets[e]) + c * B, min(B, n - c * B), c))
    vinfo = np.array(vinfo, dtype=np.int32).reshape(-1, 4)
    return {
        "counts": counts,
        "offsets": offsets.astype(np.int32),
        "sorted_slot": sorted_slot,
        "expanded_idx": expanded,
        "vinfo": vinfo,
        "num_v": int(vinfo.shape[0]),
    }


def gate_word(counts: np.ndarray, force_path: int = -1, tau: int = GATE_TAU):
    """Dense-vs-split GEMM2 decision from the sorted per-expert counts.

    [GATE] sections 1-2: one small kernel reads the sorted table after the
    sort and chooses the Split or the Dense GEMM2; the other path's kernels
    still launch and find zero items. The rule itself is not on the page;
    this reading takes Dense when the rows per touched expert reach tau.
    force_path 0/1 overrides the choice (used to test both paths).
    Returns (path, touched experts U, rows R, dense tiles or 0).
    """
    counts = np.asarray(counts, dtype=np.int64)
    U = int(np.count_nonzero(counts))
    R = int(counts.sum())
    path = 1 if (U > 0 and R >= tau * U) else 0
    if force_path in (0, 1):
        path = force_path
    ntiles = int(((counts + DENSE_MT - 1) // DENSE_MT).sum()) if path == 1 else 0
    return (path, U, R, ntiles)


def dense_tiles(counts: np.ndarray, offsets: np.ndarray, mt: int = DENSE_MT) -> np.ndarray:
    """Per-expert row tiles of the dense GEMM2 path: (expert, first_row, rows, m)."""
    out = []
    for e in np.nonzero(counts)[0]:
        n = int(counts[e])
        for m in range((n + mt - 1) // mt):
            out.append((int(e), int(offsets[e]) + m * mt, min(mt, n - m * mt), m))
    return np.array(out, dtype=np.int32).reshape(-1, 4)


def situ(g: np.ndarray, u: np.ndarray, beta: float, linear_beta: float) -> np.ndarray:
    """SiTU activation of the gate half g and the up half u, float64.

    [SHAPE] section 4 gives SiTU as the activation of the K3.1 decode kernel,
    printed only for beta = 4, linear beta = 25: the gate factor
    2 tanh(g/4) (1 + tanh(g/2)) and the up factor 25 tanh(u/25), multiplied.
    Since 1 + tanh(v/2) = 2 sigmoid(v), the gate factor is
    beta tanh(g/beta) sigmoid(g): SiLU with its linear factor g soft-capped
    at beta by tanh (beta -> infinity gives g sigmoid(g)). Reading for other
    constants: the sigmoid does not depend on beta, and the up factor is
    linear_beta tanh(u / linear_beta).
    """
    return (beta * np.tanh(g / beta) * _sigmoid(g)) * (linear_beta * np.tanh(u / linear_beta))


def expert_glu(xr: np.ndarray, W13: np.ndarray, W2: np.ndarray, limit: float = 0.0,
               act_quant: str = "bf16", act: str = "swiglu", beta: float = 4.0,
               linear_beta: float = 25.0) -> np.ndarray:
    """One expert's gated MLP on its rows, float64.

    [CUTLASS] sections 4 (GEMM1 output is (rows, 2n); SiLU on the first half
    times the second half) and the structure diagram (GEMM2 against the
    (n, k) expert weight): h = xr W13^T, g = h[:, :I], u = h[:, I:],
    act = silu(g) * u, y = act W2^T.
    With limit > 0 the clamped SwiGLU of [SHAPE] section 4 and the Marlin
    page's swiglu limit: g = min(g, limit), u = clip(u, -limit, limit).
    With act = "situ" the activation is situ(g, u, beta, linear_beta)
    instead (the limit does not apply).
    With act_quant "mxfp8" or "mxfp4" the activation is quantised to that
    MX format along I before GEMM2 ("bf16": not quantised; the oracle does
    not round it).
    xr [n, H], W13 [2I, H], W2 [H, I] -> y [n, H].
    """
    I = W13.shape[0] // 2
    h = xr @ W13.T
    g, u = h[:, :I], h[:, I:]
    if act == "situ":
        act = situ(g, u, beta, linear_beta)
    else:
        if limit > 0:
            g = np.minimum(g, limit)
            u = np.clip(u, -limit, limit)
        act = g * _sigmoid(g) * u
    if act_quant in _ACT_QUANT:
        quant, dequant = _ACT_QUANT[act_quant]
        act = dequant(*quant(act))
    return act @ W2.T


def _act_kw(s) -> dict:
    """The shape's activation as expert_glu keyword arguments."""
    return dict(act=s.activation, beta=s.act_beta, linear_beta=s.act_linear_beta)


def _routing(shape, inp):
    """Routed + shared columns: (route_ids or None, slot_expert [T,K'], slot_w [T,K'])."""
    s = shape
    T = s.T
    if s.mode == "logits":
        ids, w = route_topk_softmax(inp["logits"], s.topk)
    else:
        ids = np.asarray(inp["topk_ids"], dtype=np.int32)
        w = np.asarray(inp["topk_w"], dtype=np.float32).astype(np.float64)
    slot_expert = np.empty((T, s.Kp), dtype=np.int32)
    slot_w = np.empty((T, s.Kp), dtype=np.float64)
    slot_expert[:, : s.topk] = local_map(ids, s.E, s.expert_offset)
    slot_w[:, : s.topk] = w
    if s.S > 0:
        sid, sw = shared_append(inp["shared"], s.E, s.S, s.shared_scale)
        slot_expert[:, s.topk:] = sid
        slot_w[:, s.topk:] = sw
    return ids, slot_expert, slot_w


def _activations(shape, inp):
    """x as GEMM1 reads it: bf16 values, or their MX quantisation along H
    (returned with its codes and scales)."""
    x = bf16_bits_to_f64(inp["x"])
    if shape.a_dtype in _ACT_QUANT:
        quant, dequant = _ACT_QUANT[shape.a_dtype]
        xq, xs = quant(x)
        return dequant(xq, xs), xq, xs
    return x, None, None


def reference_forward(shape, inp: dict, force_path: int = -1, compute_out: bool = True) -> dict:
    """The whole layer on all tokens, float64 (no rounding anywhere).

    Routing, shared append, local map, sort and gate as above; then, per
    touched expert, the gathered rows go through expert_glu and the result is
    added into the token's output times its routing weight: the
    shuffle-mul-sum of [CUTLASS] section 5, skipping -1 slots ([SHAPE]
    section 5). Tokens with no local slot get exact zeros.
    Returns the maps and out [T, H] float64 (if compute_out).
    """
    s = shape
    ids, slot_expert, slot_w = _routing(s, inp)
    maps = sort_align(slot_expert, s.Ep, s.B)
    gate = gate_word(maps["counts"], force_path)
    res = dict(maps)
    res.update(route_ids=ids, slot_expert=slot_expert, slot_w=slot_w, gate=gate,
               kmax_v=kmax_v(s.Ep, s.T, s.Kp, s.B))
    res["dense_tiles"] = dense_tiles(maps["counts"], maps["offsets"]) if gate[0] == 1 \
        else np.zeros((0, 4), np.int32)
    xa, xq, xs = _activations(s, inp)
    res["xq"], res["xs"] = xq, xs
    if not compute_out:
        return res
    out = np.zeros((s.T, s.H), dtype=np.float64)
    counts, offsets, sorted_slot = maps["counts"], maps["offsets"], maps["sorted_slot"]
    wflat = slot_w.reshape(-1)
    for e in np.nonzero(counts)[0]:
        rows = sorted_slot[offsets[e]: offsets[e + 1]].astype(np.int64)
        tok = rows // s.Kp
        W13 = dequant_mxfp4(inp["w13"][e], inp["s13"][e])
        W2 = dequant_mxfp4(inp["w2"][e], inp["s2"][e])
        y = expert_glu(xa[tok], W13, W2, s.swiglu_limit, s.a_dtype, **_act_kw(s))
        np.add.at(out, tok, wflat[rows][:, None] * y)
    res["out"] = out
    return res


def sampled_forward(shape, inp: dict, tokens) -> np.ndarray:
    """Output rows of the given tokens, computed one token at a time.

    No sort and no grouping: for each token, each of its columns with a
    local expert runs that expert's gated MLP on the token alone and adds
    weight * result. Equals reference_forward(...)["out"][tokens]; cheap
    enough to check a sample of a full-size layer.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    s = shape.replace(T=int(tokens.shape[0]))
    sub = {k: np.asarray(inp[k])[tokens] for k in ("x", "logits", "shared", "topk_ids", "topk_w")
           if k in inp}
    ids, slot_expert, slot_w = _routing(s, sub)
    xa, _, _ = _activations(s, sub)
    cache: dict = {}
    out = np.zeros((tokens.shape[0], s.H), dtype=np.float64)
    for i in range(tokens.shape[0]):
        for k in range(s.Kp):
            e = int(slot_expert[i, k])
            if e < 0:
                continue
            if e not in cache:
                cache[e] = (dequant_mxfp4(inp["w13"][e], inp["s13"][e]),
                            dequant_mxfp4(inp["w2"][e], inp["s2"][e]))
            W13, W2 = cache[e]
            y = expert_glu(xa[i: i + 1], W13, W2, s.swiglu_limit, s.a_dtype, **_act_kw(s))
            out[i] += slot_w[i, k] * y[0]
    return out
