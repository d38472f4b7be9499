"""Python binding of libmoe_mxfp4 (the fused MXFP4 MoE layer for MI355X).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The names
mirror the C ABI in include/moe_mxfp4.h: query, workspace_layout, forward,
strerror. There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = ["Shape", "query", "workspace_layout", "forward", "forward_timed", "forward_noalloc",
           "strerror", "lib_path", "MoeError", "read_maps", "ADTYPE", "GEMM2_PATH", "load_library",
           "prepack"]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_OK = 0
NUM_STAGES = 5  # route, sort + gate, GEMM1, GEMM2, finalize
STAGE_NAMES = ("route", "sort_gate", "gemm1", "gemm2", "finalize")
ADTYPE = {"bf16": 0, "mxfp8": 1, "mxfp4": 2}
ACTIVATION = {"swiglu": 0, "situ": 1}
GEMM2_PATH = {"auto": -1, "split": 0, "dense": 1}
WEIGHT_LAYOUT = {"row_major": 0, "packed": 1}


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "E", "E_global", "topk", "S", "H", "I", "block_n", "expert_offset", "activation",
        "a_dtype", "force_gemm2_path")] + [("swiglu_limit", ctypes.c_float),
                                            ("shared_scale", ctypes.c_float),
                                            ("act_beta", ctypes.c_float),
                                            ("act_linear_beta", ctypes.c_float),
                                            ("weight_layout", ctypes.c_int32)]


_LAYOUT_U64 = ("total_bytes", "counters", "route_ids", "slot_expert", "slot_w", "range_counts",
               "counts", "offsets", "sorted_slot", "expanded_idx", "vinfo", "dense_tiles", "units16", "act",
               "act_scales", "y", "xq", "xs")
_LAYOUT_I32 = ("kmax_v", "max_dense_tiles", "max_units16", "n_ranges", "rows_pad")


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in _LAYOUT_U64] + [(n, ctypes.c_int32) for n in _LAYOUT_I32]


_lib = None


def load_library():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build it with "
                           "`python -m mxfp4_weight_expert_amd.build`")
    lib = ctypes.CDLL(lib_path)
    lib.moe_mxfp4_query.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(ctypes.c_uint64)]
    lib.moe_mxfp4_query.restype = ctypes.c_int
    lib.moe_mxfp4_workspace_layout.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(_Layout)]
    lib.moe_mxfp4_workspace_layout.restype = ctypes.c_int
    lib.moe_mxfp4_strerror.argtypes = [ctypes.c_int]
    lib.moe_mxfp4_strerror.restype = ctypes.c_char_p
    vp = ctypes.c_void_p
    lib.moe_mxfp4_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Shape),
                                      vp, vp, ctypes.c_uint64, vp]
    lib.moe_mxfp4_forward.restype = ctypes.c_int
    lib.moe_mxfp4_forward_timed.argtypes = lib.moe_mxfp4_forward.argtypes + [ctypes.c_void_p]
    lib.moe_mxfp4_forward_timed.restype = ctypes.c_int
    lib.moe_mxfp4_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.POINTER(_Shape), vp, vp]
    lib.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
    lib.moe_mxfp4_prepack.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
    lib.moe_mxfp4_prepack.restype = ctypes.c_int
    _lib = lib
    return lib


@dataclass(frozen=True)
class Shape:
    """Layer shape (fields as in moe_mxfp4_shape)."""

    T: int
    E: int
    E_global: int
    topk: int
    H: int
    I: int
    block_n: int
    S: int = 0
    expert_offset: int = 0
    swiglu_limit: float = 0.0
    shared_scale: float = 1.0
    a_dtype: str = "bf16"
    force_gemm2_path: str = "auto"
    activation: str = "swiglu"  # or "situ"
    act_beta: float = 4.0  # SiTU caps (read only for "situ")
    act_linear_beta: float = 25.0
    weight_layout: str = "packed"  # w13/w2 as prepack() returns them

    def to_c(self) -> _Shape:
        return _Shape(self.T, self.E, self.E_global, self.topk, self.S, self.H, self.I,
                      self.block_n, self.expert_offset, ACTIVATION[self.activation],
                      ADTYPE[self.a_dtype], GEMM2_PATH[self.force_gemm2_path],
                      float(self.swiglu_limit), float(self.shared_scale), float(self.act_beta),
                      float(self.act_linear_beta), WEIGHT_LAYOUT[self.weight_layout])

    @property
    def Kp(self) -> int:
        return self.topk + self.S

    @property
    def Ep(self) -> int:
        return self.E + self.S


def strerror(code: int) -> str:
    return load_library().moe_mxfp4_strerror(code).decode()


def query(shape: Shape) -> int:
    """Workspace bytes for a shape (raises MoeError if unsupported)."""
    n = ctypes.c_uint64()
    rc = load_library().moe_mxfp4_query(ctypes.byref(shape.to_c()), ctypes.byref(n))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_mxfp4_query")
    return int(n.value)


def workspace_layout(shape: Shape) -> dict:
    lay = _Layout()
    rc = load_library().moe_mxfp4_workspace_layout(ctypes.byref(shape.to_c()), ctypes.byref(lay))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_mxfp4_workspace_layout")
    return {n: int(getattr(lay, n)) for n in _LAYOUT_U64 + _LAYOUT_I32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(fn, x, w13, s13, w2, s2, shape, router_logits, topk_ids, topk_w, shared_logits, out,
          workspace, stream, extra):
    import torch

    for t in (x, w13, s13, w2, s2, router_logits, topk_ids, topk_w, shared_logits, out, workspace):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(query(shape), 256), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = fn(_ptr(x), _ptr(router_logits), _ptr(topk_ids), _ptr(topk_w), _ptr(shared_logits),
            _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), ctypes.byref(shape.to_c()), _ptr(out),
            _ptr(workspace), ctypes.c_uint64(workspace.numel()), ctypes.c_void_p(stream), *extra)
    if rc != MOE_OK:
        raise MoeError(rc, fn.__name__)
    return out


def prepack(w, rows: int = None, out=None, stream=None):
    """Weights in the packed layout the forward calls read (moe_mxfp4_prepack).

    w: contiguous uint8 device tensor, a row-major matrix of `rows` rows
    (default: the product of all but the last dimension) of nibble-packed
    E2M1 codes, e.g. w13 [E', 2I, H/2] or w2 [E', H, I/2]. Returns a new
    tensor of the same shape (or fills `out`)."""
    import torch

    if not w.is_contiguous() or w.dtype != torch.uint8:
        raise ValueError("w must be a contiguous uint8 tensor")
    row_bytes = w.shape[-1]
    if rows is None:
        rows = w.numel() // row_bytes
    if out is None:
        out = torch.empty_like(w)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    rc = load_library().moe_mxfp4_prepack(_ptr(w), _ptr(out), ctypes.c_int64(rows),
                                          ctypes.c_int64(row_bytes), ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_mxfp4_prepack")
    return out


def forward(x, w13, s13, w2, s2, shape: Shape, *, router_logits=None, topk_ids=None, topk_w=None,
            shared_logits=None, out=None, workspace=None, stream=None):
    """Run the layer; returns out (bf16 [T, H]).

    x bf16 [T, H]; w13/s13/w2/s2 uint8 as in the C header (w13 and w2 in
    the packed layout of prepack); router_logits
    float32 [T, E_global] or (topk_ids int32 [T, topk], topk_w float32
    [T, topk]); shared_logits bf16 [T, S]. workspace: a uint8 CUDA tensor of
    at least query(shape) bytes (allocated here when None). All tensors must
    be contiguous and on the current device.
    """
    return _call(load_library().moe_mxfp4_forward, x, w13, s13, w2, s2, shape, router_logits,
                 topk_ids, topk_w, shared_logits, out, workspace, stream, ())


NOALLOC_SCRATCH_BYTES = 128 << 20


def forward_noalloc(x, w13, s13, w2, s2, shape: Shape, *, router_logits=None, topk_ids=None,
                    topk_w=None, shared_logits=None, out=None, stream=None):
    """forward through moe_mxfp4_forward_noalloc: no workspace argument, the
    library's per-GPU scratch array instead (shapes up to
    NOALLOC_SCRATCH_BYTES of workspace). `out` must be given by callers that
    cannot allocate; it is allocated here when None."""
    import torch

    for t in (x, w13, s13, w2, s2, router_logits, topk_ids, topk_w, shared_logits, out):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    fn = load_library().moe_mxfp4_forward_noalloc
    rc = fn(_ptr(x), _ptr(router_logits), _ptr(topk_ids), _ptr(topk_w), _ptr(shared_logits),
            _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), ctypes.byref(shape.to_c()), _ptr(out),
            ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_mxfp4_forward_noalloc")
    return out


def forward_timed(events, x, w13, s13, w2, s2, shape: Shape, *, router_logits=None, topk_ids=None,
                  topk_w=None, shared_logits=None, out=None, workspace=None, stream=None):
    """forward, recording NUM_STAGES + 1 torch.cuda.Event objects (enable_timing=True)
    between the stages of the launch chain on the library's stream."""
    if len(events) != NUM_STAGES + 1:
        raise ValueError(f"need {NUM_STAGES + 1} events")
    for e in events:
        if not e.cuda_event:  # torch creates the HIP event on its first record
            e.record()
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    return _call(load_library().moe_mxfp4_forward_timed, x, w13, s13, w2, s2, shape,
                 router_logits, topk_ids, topk_w, shared_logits, out, workspace, stream, (arr,))


def read_maps(workspace, shape: Shape) -> dict:
    """Views of the maps a forward call left in the workspace (device tensors)."""
    import torch

    L = workspace_layout(shape)
    T, Kp, Ep = shape.T, shape.Kp, shape.Ep

    def view(off, n, dtype):
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return workspace[off: off + nbytes].view(dtype)

    i32, f32 = torch.int32, torch.float32
    ctr = view(L["counters"], 64, i32)
    maps = {
        "counters": ctr,
        "route_ids": view(L["route_ids"], T * shape.topk, i32).view(T, shape.topk),
        "slot_expert": view(L["slot_expert"], T * Kp, i32).view(T, Kp),
        "slot_w": view(L["slot_w"], T * Kp, f32).view(T, Kp),
        "counts": view(L["counts"], Ep, i32),
        "offsets": view(L["offsets"], Ep + 1, i32),
        "sorted_slot": view(L["sorted_slot"], T * Kp, i32),
        "expanded_idx": view(L["expanded_idx"], T * Kp, i32),
        "vinfo": view(L["vinfo"], L["kmax_v"] * 4, i32).view(-1, 4),
        "dense_tiles": view(L["dense_tiles"], L["max_dense_tiles"] * 4, i32).view(-1, 4),
        "units16": view(L["units16"], L["max_units16"] * 4, i32).view(-1, 4),
        "act": view(L["act"], L["rows_pad"] * shape.I * {"bf16": 4, "mxfp8": 2, "mxfp4": 1}[
            shape.a_dtype] // 2, torch.uint8),
        "y": view(L["y"], L["rows_pad"] * shape.H, torch.bfloat16).view(L["rows_pad"], shape.H),
        "layout": L,
    }
    if shape.a_dtype in ("mxfp8", "mxfp4"):
        xb = shape.H if shape.a_dtype == "mxfp8" else shape.H // 2  # code bytes per row
        maps["xq"] = view(L["xq"], T * xb, torch.uint8).view(T, xb)
        maps["xs"] = view(L["xs"], T * shape.H // 32, torch.uint8).view(T, shape.H // 32)
        maps["act_scales"] = view(L["act_scales"], L["rows_pad"] * shape.I // 32, torch.uint8)
    return maps
