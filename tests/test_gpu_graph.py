"""The launch chain under hipGraph capture: one graph, captured once, serves
every input. The GEMM2 path is chosen on the device from the routing, so a
replay must follow new router logits written into the captured buffers, also
when they flip the gate between the split and the dense path. Each replay is
compared bit for bit with an eager call on the same inputs, and those eager
outputs with the fp64 oracle; the replays are separated by eager copies and
synchronisations.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_weight_expert_amd as moe
from workloads import LayerShape, make_inputs

from gpu_util import check_maps, check_out, lib_shape, maps_np, out_np, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("a_dtype", ["bf16", "mxfp8", "mxfp4"])
def test_graph_replay_follows_inputs_across_the_gate(a_dtype):
    s = LayerShape("graph_gate", T=256, E=64, E_g=64, topk=4, H=512, I=128, B=32, a_dtype=a_dtype)
    inp = make_inputs(s, 777)
    spread = inp["logits"]                     # 1,024 rows over ~64 experts: split path
    conc = spread.copy()
    conc[:, :4] += np.float32(100.0)           # every token picks experts 0..3: dense path
    sets = {"spread": spread, "conc": conc}

    dev = to_device(s, inp)
    logits = dev["logits"]                     # the buffer the graph reads
    shp = lib_shape(s)
    nbytes = moe.query(shp)

    def call(out, ws):
        moe.forward(dev["x"], dev["w13"], dev["s13"], dev["w2"], dev["s2"], shp,
                    router_logits=logits, out=out, workspace=ws)

    def bits(t):
        torch.cuda.synchronize()
        return t.view(torch.int16).cpu().numpy()

    # eager references, each checked against the oracle
    ws_e = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out_e = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    want, paths = {}, {}
    for name, lg in sets.items():
        say(f"[graph] eager {name} a_dtype={a_dtype}")
        logits.copy_(torch.from_numpy(lg))
        call(out_e, ws_e)
        ref = oracle.reference_forward(s, dict(inp, logits=lg))
        check_maps(s, maps_np(s, ws_e), ref)
        check_out(out_np(out_e), ref["out"], f"graph_gate/{name}/eager")
        want[name] = bits(out_e)
        paths[name] = int(ref["gate"][0])
    assert paths == {"spread": 0, "conc": 1}

    # one capture on a side stream, then replays over both routings
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    call(out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        call(out, ws)
    torch.cuda.synchronize()
    for i, name in enumerate(["spread", "conc", "conc", "spread", "conc", "spread"]):
        say(f"[graph] replay {i}: {name}")
        logits.copy_(torch.from_numpy(sets[name]))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(bits(out), want[name]), f"replay {i} ({name}) differs from eager"
        gate = int(maps_np(s, ws)["counters"][4])
        assert gate == paths[name], f"replay {i} ({name}): gate path {gate}"
