"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, agrees with the header on struct layout,
and rejects bad arguments before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

import mxfp4_weight_expert_amd as moe
import oracle
from workloads import CONFIGS, CONFIG_ORDER

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_mxfp4_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = moe.load_library()
    names = _declared_functions()
    assert names == ["moe_mxfp4_forward", "moe_mxfp4_forward_noalloc", "moe_mxfp4_forward_timed",
                     "moe_mxfp4_prepack", "moe_mxfp4_query", "moe_mxfp4_strerror",
                     "moe_mxfp4_workspace_layout"]
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", moe.lib_path], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (moe_mxfp4_\w+)", nm.stdout))
    assert exported == set(names)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "probe.c"
    fields_s = [f[0] for f in moe._Shape._fields_]
    fields_l = [f[0] for f in moe._Layout._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe_mxfp4.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(moe_mxfp4_shape), sizeof(moe_mxfp4_ws_layout));']
    lines += [f'printf("%zu\\n", offsetof(moe_mxfp4_shape, {f}));' for f in fields_s]
    lines += [f'printf("%zu\\n", offsetof(moe_mxfp4_ws_layout, {f}));' for f in fields_l]
    lines += ["return 0;}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(moe._Shape) and vals[1] == ctypes.sizeof(moe._Layout)
    offs = [getattr(moe._Shape, f).offset for f in fields_s] + \
           [getattr(moe._Layout, f).offset for f in fields_l]
    assert vals[2:] == offs


def _shape(**kw):
    base = dict(T=64, E=896, E_global=896, topk=16, H=3584, I=384, block_n=32)
    base.update(kw)
    return moe.Shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(H=3584 + 256), 2), (dict(I=384 + 64), 2), (dict(block_n=48), 2), (dict(topk=33), 2),
    (dict(S=9), 2), (dict(E=2040, E_global=2040, S=9), 2), (dict(E_global=3000, E=2000), 2),
    (dict(expert_offset=1), 1), (dict(T=-1), 1), (dict(E=0), 1), (dict(topk=0), 1),
    (dict(force_gemm2_path="dense", T=1 << 20), 2), (dict(H=8192 + 512), 2), (dict(I=8192 + 128), 2),
    (dict(activation="situ", act_beta=0.0), 1), (dict(activation="situ", act_linear_beta=-1.0), 1),
    (dict(activation="situ", act_beta=float("inf")), 1),
    (dict(activation="situ", act_linear_beta=float("nan")), 1),
])
def test_query_rejects_bad_shapes(kw, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.query(_shape(**kw))
    assert ei.value.code == code


def test_query_activation_kinds():
    assert moe.query(_shape(activation="situ")) == moe.query(_shape())
    # the SiTU caps are not read for SwiGLU
    assert moe.query(_shape(act_beta=0.0, act_linear_beta=float("nan"))) > 0
    bad = _shape().to_c()
    bad.activation = 2
    n = ctypes.c_uint64()
    assert moe.load_library().moe_mxfp4_query(ctypes.byref(bad), ctypes.byref(n)) == 2


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_layout_bounds_match_oracle(name):
    s = CONFIGS[name]
    L = moe.workspace_layout(moe.Shape(T=s.T, E=s.E, E_global=s.E_g, topk=s.topk, H=s.H, I=s.I,
                                       block_n=s.B, S=s.S, expert_offset=s.expert_offset))
    assert L["kmax_v"] == oracle.kmax_v(s.Ep, s.T, s.Kp, s.B)
    offs = [L[k] for k in ("counters", "route_ids", "slot_expert", "slot_w", "range_counts",
                           "counts", "offsets", "sorted_slot", "expanded_idx", "vinfo",
                           "dense_tiles", "units16", "act", "act_scales", "y", "xq", "xs")]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and offs[-1] <= L["total_bytes"]
    assert L["y"] - L["act"] >= L["rows_pad"] * s.I * 2
    assert L["total_bytes"] - L["y"] >= L["rows_pad"] * s.H * 2
    assert L["rows_pad"] >= s.T * s.Kp


def test_kimi_k31_virtual_expert_bound_from_layout():
    L = moe.workspace_layout(_shape(T=256, block_n=32))
    assert L["kmax_v"] == 1024


def _no_device():
    """True when no HIP device is visible. Counting devices does not
    initialise the GPU. The rejection tests below pass fabricated device
    addresses: they must never run where a kernel could be dispatched if a
    validation check regressed."""
    import torch
    return torch.cuda.device_count() == 0


fabricated_addresses = pytest.mark.skipif(
    not _no_device(), reason="fabricated device addresses: run only where no GPU is visible")


def _fwd(shape, logits=1024, ids=None, w=None, ws=256, wsb=1 << 40, shared=None, x=256, w13=256,
         s13=256, w2=256, s2=256, out=256):
    """moe_mxfp4_forward on fake device addresses: only calls that fail
    validation before any launch may be made here."""
    lib = moe.load_library()
    P = ctypes.c_void_p
    return lib.moe_mxfp4_forward(P(x), P(logits) if logits else None, P(ids) if ids else None,
                                 P(w) if w else None, P(shared) if shared else None, P(w13), P(s13),
                                 P(w2), P(s2), ctypes.byref(shape.to_c()), P(out),
                                 P(ws) if ws else None, ctypes.c_uint64(wsb), None)


@fabricated_addresses
def test_forward_rejects_before_launch():
    s = _shape()
    assert _fwd(s, logits=1024, ids=512, w=512) == 1    # both routing inputs
    assert _fwd(s, logits=None) == 1                     # neither
    assert _fwd(s, logits=None, ids=512) == 1            # ids without weights
    assert _fwd(s, wsb=1024) == 3                        # workspace too small
    assert _fwd(s, ws=256 + 64) == 3                     # misaligned workspace
    assert _fwd(s, ws=None) == 1
    assert _fwd(_shape(S=1), shared=None) == 1           # shared experts need logits
    assert _fwd(_shape(H=100)) == 2
    assert _fwd(_shape(T=0), ws=None) == 0               # empty call: nothing to do
    # misaligned buffers (each valid otherwise: the workspace is too small,
    # so an aligned call would stop at MOE_ERR_WORKSPACE before any launch)
    assert _fwd(s, wsb=1024) == 3
    for kw in ({"x": 264}, {"out": 264}, {"w13": 260}, {"s13": 264}, {"w2": 258}, {"s2": 260},
               {"logits": 1026}):
        assert _fwd(s, wsb=1024, **kw) == 1, kw
    assert _fwd(s, wsb=1024, logits=None, ids=514, w=512) == 1
    assert _fwd(s, wsb=1024, logits=None, ids=512, w=514) == 1
    assert _fwd(_shape(S=1), wsb=1024, shared=513) == 1
    assert _fwd(_shape(S=1), wsb=1024, shared=514) == 3  # 2-byte aligned is enough


@fabricated_addresses
def test_forward_rejects_row_major_weights_before_launch():
    # a valid call in every other respect (workspace large enough, aligned):
    # the row-major tag alone stops it
    assert _fwd(_shape(weight_layout="row_major")) == 2
    assert _fwd(_shape(weight_layout="row_major"), ws=None) == 2  # before the pointer checks
    assert _fwd(_shape(T=0, weight_layout="row_major"), ws=None) == 2
    bad = _shape().to_c()
    bad.weight_layout = 7
    lib = moe.load_library()
    P = ctypes.c_void_p
    assert lib.moe_mxfp4_forward(P(256), P(1024), None, None, None, P(256), P(256), P(256), P(256),
                                 ctypes.byref(bad), P(256), P(256), ctypes.c_uint64(1 << 40),
                                 None) == 1


def test_weight_layout_tag_in_query():
    # query and workspace_layout read no weights: both tags give the same size
    assert moe.query(_shape(weight_layout="row_major")) == moe.query(_shape())
    bad = _shape().to_c()
    bad.weight_layout = -1
    n = ctypes.c_uint64()
    assert moe.load_library().moe_mxfp4_query(ctypes.byref(bad), ctypes.byref(n)) == 1


@fabricated_addresses
def test_prepack_rejects_before_launch():
    lib = moe.load_library()
    P = ctypes.c_void_p

    def pk(src, dst, rows, row_bytes):
        return lib.moe_mxfp4_prepack(P(src) if src else None, P(dst) if dst else None,
                                     ctypes.c_int64(rows), ctypes.c_int64(row_bytes), None)

    assert pk(None, 1 << 20, 16, 64) == 1                # null source
    assert pk(1 << 20, None, 16, 64) == 1                # null destination
    assert pk(1 << 20, (1 << 20) + 8, 16, 64) == 1       # misaligned destination
    assert pk(1 << 20, (1 << 20) + 512, 16, 64) == 1     # overlapping buffers
    assert pk(1 << 20, 1 << 24, 0, 64) == 1              # no rows
    assert pk(1 << 20, 1 << 24, 8, 64) == 2              # rows not a multiple of 16
    assert pk(1 << 20, 1 << 24, 16, 48) == 2             # row bytes not a multiple of 64


def test_strerror():
    assert moe.strerror(0) == "ok"
    assert "workspace" in moe.strerror(3)
    assert moe.strerror(99) == "unknown error"
