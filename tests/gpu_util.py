"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mxfp4_weight_expert_amd as moe
import oracle
from workloads import LayerShape

# Output tolerances: max |got - want| / max |want| and ||got - want|| / ||want||.
MAXABS_NORM_TOL = 2e-2
REL_L2_TOL = 5e-3
# Routing weights: fp32 on the GPU vs fp64 in the oracle.
WEIGHT_RTOL = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def lib_shape(s: LayerShape, force: str = "auto") -> moe.Shape:
    return moe.Shape(T=s.T, E=s.E, E_global=s.E_g, topk=s.topk, H=s.H, I=s.I, block_n=s.B, S=s.S,
                     expert_offset=s.expert_offset, swiglu_limit=s.swiglu_limit,
                     shared_scale=s.shared_scale, a_dtype=s.a_dtype, force_gemm2_path=force,
                     activation=s.activation, act_beta=s.act_beta,
                     act_linear_beta=s.act_linear_beta)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_device(s: LayerShape, inp: dict) -> dict:
    d = {
        "x": bf16_dev(inp["x"]),
        "w13": moe.prepack(torch.from_numpy(inp["w13"]).cuda()),
        "s13": torch.from_numpy(inp["s13"]).cuda(),
        "w2": moe.prepack(torch.from_numpy(inp["w2"]).cuda()),
        "s2": torch.from_numpy(inp["s2"]).cuda(),
        "shared": bf16_dev(inp["shared"]) if s.S > 0 else None,
    }
    if s.mode == "ids":
        d["topk_ids"] = torch.from_numpy(inp["topk_ids"]).cuda()
        d["topk_w"] = torch.from_numpy(inp["topk_w"]).cuda()
    else:
        d["logits"] = torch.from_numpy(inp["logits"]).cuda()
    return d


def run(s: LayerShape, dev: dict, force: str = "auto", workspace=None, out=None):
    """One forward call; returns (out tensor, workspace tensor)."""
    shp = lib_shape(s, force)
    if workspace is None:
        workspace = torch.empty(max(moe.query(shp), 256), dtype=torch.uint8, device="cuda")
    out = moe.forward(dev["x"], dev["w13"], dev["s13"], dev["w2"], dev["s2"], shp,
                      router_logits=dev.get("logits"), topk_ids=dev.get("topk_ids"),
                      topk_w=dev.get("topk_w"), shared_logits=dev.get("shared"),
                      workspace=workspace, out=out)
    return out, workspace


def maps_np(s: LayerShape, workspace, force: str = "auto") -> dict:
    m = moe.read_maps(workspace, lib_shape(s, force))
    torch.cuda.synchronize()
    out = {}
    for k, v in m.items():
        if isinstance(v, torch.Tensor) and k not in ("act", "y"):
            out[k] = v.cpu().numpy()
    return out


def out_np(out: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check_out(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Normalised max-abs and relative L2 against the fp64 oracle."""
    amax = float(np.max(np.abs(want))) if want.size else 0.0
    if amax == 0.0:
        assert np.all(got == 0), f"{what}: expected exact zeros"
        return 0.0, 0.0
    err = got - want
    mx = float(np.max(np.abs(err))) / amax
    rl2 = float(np.linalg.norm(err) / np.linalg.norm(want))
    say(f"  {what}: max|err|/max|ref| = {mx:.2e}  relL2 = {rl2:.2e}  (max|ref| = {amax:.3g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= MAXABS_NORM_TOL, f"{what}: normalised max-abs {mx:.3e} > {MAXABS_NORM_TOL}"
    assert rl2 <= REL_L2_TOL, f"{what}: rel-L2 {rl2:.3e} > {REL_L2_TOL}"
    return mx, rl2


def check_maps(s: LayerShape, got: dict, ref: dict, force_path: int = -1):
    """Integer maps bit-exact; routing weights to WEIGHT_RTOL."""
    if s.mode == "logits":
        assert np.array_equal(got["route_ids"], ref["route_ids"]), "top-k ids differ"
    assert np.array_equal(got["slot_expert"], ref["slot_expert"]), "slot experts differ"
    assert np.allclose(got["slot_w"], ref["slot_w"], rtol=WEIGHT_RTOL, atol=0, equal_nan=True), \
        "slot weights differ"
    assert np.array_equal(got["counts"], ref["counts"]), "counts differ"
    assert np.array_equal(got["offsets"], ref["offsets"]), "offsets differ"
    R = int(ref["counts"].sum())
    assert np.array_equal(got["sorted_slot"][:R], ref["sorted_slot"]), "sorted_slot differs"
    assert np.array_equal(got["expanded_idx"], ref["expanded_idx"]), "expanded_idx differs"
    nv = int(got["counters"][0])
    assert nv == ref["num_v"], f"num_v {nv} != {ref['num_v']}"
    assert nv <= ref["kmax_v"]
    assert np.array_equal(got["vinfo"][:nv], ref["vinfo"]), "chunk table differs"
    gate = tuple(int(v) for v in got["counters"][4:8])
    assert gate == tuple(ref["gate"]), f"gate word {gate} != {ref['gate']}"
    nt = gate[3]
    assert np.array_equal(got["dense_tiles"][:nt], ref["dense_tiles"]), "dense tiles differ"
    nu = int(got["counters"][1])
    u16 = oracle.sort_align(ref["slot_expert"], s.Ep, 16)["vinfo"]
    assert nu == u16.shape[0] and np.array_equal(got["units16"][:nu], u16), "16-row units differ"


def covering_tokens(ref: dict, Kp: int, B: int, tile: int) -> np.ndarray:
    """Tokens whose rows cover, from the oracle's maps, (a) the last B-row
    chunk (the ragged tail) of every expert with rows, and (b) every row
    position 0..tile-1 within an expert's tile-row tiles (the last slot of a
    tile included). Greedy: the token of each uncovered expert's last row,
    then a token for each position still uncovered."""
    offsets = ref["offsets"].astype(np.int64)
    counts = ref["counts"].astype(np.int64)
    sorted_slot = ref["sorted_slot"].astype(np.int64)
    expanded = ref["expanded_idx"].astype(np.int64)
    R = int(counts.sum())
    rows_all = np.arange(R)
    row_expert = np.searchsorted(offsets, rows_all, side="right") - 1
    pos = rows_all - offsets[row_expert]
    tail_start = offsets[:-1] + (np.maximum(counts, 1) - 1) // B * B
    in_tail = rows_all >= tail_start[row_expert]
    tail_done = counts == 0
    pos_done = np.zeros(tile, bool)
    chosen = []

    def take(t):
        chosen.append(t)
        rows = expanded[t * Kp:(t + 1) * Kp]
        rows = rows[rows >= 0]
        tail_done[row_expert[rows[in_tail[rows]]]] = True
        pos_done[pos[rows] % tile] = True

    for e in np.nonzero(~tail_done)[0]:
        if not tail_done[e]:
            take(int(sorted_slot[offsets[e + 1] - 1]) // Kp)
    for p in np.nonzero(~pos_done)[0]:
        if not pos_done[p] and np.any(counts > p):
            e = int(np.argmax(counts > p))
            take(int(sorted_slot[offsets[e] + p]) // Kp)
    assert np.all(tail_done)
    return np.unique(chosen)


def oracle_rows(s: LayerShape, inp: dict, tokens: np.ndarray) -> np.ndarray:
    """The oracle's output rows for `tokens`: the whole layer on that
    sub-batch (every step is per token, so the rows equal those of the full
    batch), grouped by expert so each touched expert is decoded once."""
    sub = {k: (np.asarray(v)[tokens] if k in ("x", "logits", "shared", "topk_ids", "topk_w") else v)
           for k, v in inp.items()}
    return oracle.reference_forward(s.replace(T=int(len(tokens))), sub)["out"]
