"""The allocation-free entry point (moe_mxfp4_forward_noalloc) against the
workspace entry point (moe_mxfp4_forward): same kernels, same inputs, so the
outputs must match bit for bit; both are also checked against the fp64
oracle. Two calls in a row on the library's scratch array, the second with a
smaller input (the first call's maps stay behind in the array), then a shape
whose workspace exceeds the array, rejected before any launch."""
import numpy as np
import pytest
import torch

import mxfp4_weight_expert_amd as moe
import oracle
from workloads import LayerShape, make_inputs

from gpu_util import check_out, lib_shape, out_np, run, say, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # larger first: many chunks, a shared expert, LDS token tiles
    LayerShape("na_large", T=200, E=64, E_g=96, topk=8, H=1024, I=256, B=32, S=1,
               expert_offset=16, swiglu_limit=7.0),
    # then smaller, on the same scratch
    LayerShape("na_small", T=5, E=8, E_g=8, topk=2, H=512, I=128, B=16),
    # W4A8, many rows per expert: tiled GEMM1 and the dense GEMM2
    LayerShape("na_a8_prefill", T=700, E=6, E_g=6, topk=2, H=512, I=256, B=128, a_dtype="mxfp8"),
    LayerShape("na_tiny_again", T=3, E=4, E_g=4, topk=1, H=512, I=128, B=32),
]


def _noalloc(s, dev, out):
    return moe.forward_noalloc(dev["x"], dev["w13"], dev["s13"], dev["w2"], dev["s2"], lib_shape(s),
                               router_logits=dev.get("logits"), shared_logits=dev.get("shared"),
                               out=out)


def test_noalloc_matches_forward_on_consecutive_calls():
    for i, s in enumerate(CASES):
        say(f"[noalloc] {s.name}")
        inp = make_inputs(s, 6100 + i)
        dev = to_device(s, inp)
        want, _ = run(s, dev)
        out = torch.full((s.T, s.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = _noalloc(s, dev, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{s.name}: differs"
        check_out(out_np(got), oracle.reference_forward(s, inp)["out"], f"{s.name} noalloc")


def test_noalloc_rejects_oversized_workspace_before_launch():
    s = LayerShape("na_big", T=32768, E=8, E_g=8, topk=8, H=512, I=128, B=128)
    shp = lib_shape(s)
    assert moe.query(shp) > moe.NOALLOC_SCRATCH_BYTES
    # full-size inputs and output (small weights), so the call would stay in
    # bounds even if it were not rejected
    dev = to_device(s, make_inputs(s, 3))
    out = torch.full((s.T, s.H), 2.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(dev["x"], dev["w13"], dev["s13"], dev["w2"], dev["s2"], shp,
                            router_logits=dev["logits"], out=out)
    assert ei.value.code == 5
    torch.cuda.synchronize()
    assert bool(torch.all(out == 2.0))
