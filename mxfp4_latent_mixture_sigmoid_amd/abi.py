"""ctypes binding of the C ABI in include/mxmoe.h (argument marshalling only).

Every step of the layer runs in the HIP library ``libmxmoe.so``; this module only turns torch
tensors into device pointers and the current HIP stream into a ``hipStream_t``. If the library
is missing it raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from enum import IntEnum

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxmoe.so")

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t


class Status(IntEnum):
    OK = 0
    INVALID_ARG = -1
    UNSUPPORTED = -2
    BUFFER_TOO_SMALL = -3
    HIP = -4


ACT_SILU_GLU = 0
STAGE2_BF16 = 0
STAGE2_FP8 = 1
STAGE1_BF16 = 0
STAGE1_MXFP4 = 1
SHARED_FUSED = 0
SHARED_STREAM = 1


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("latent", c_i32), ("n_experts", c_i32), ("top_k", c_i32),
                ("inter", c_i32), ("n_shared", c_i32), ("shared_inter", c_i32),
                ("has_latent_proj", c_i32), ("act", c_i32), ("stage2", c_i32),
                ("stage1", c_i32), ("shared_stream", c_i32)]


WEIGHT_FIELDS = ("w_router", "w_down", "w_up", "gate_codes", "gate_scales", "up_codes", "up_scales",
                 "down_codes", "down_scales", "sh_gate", "sh_up", "sh_down")


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in WEIGHT_FIELDS]


ROUTING_FIELDS = ("topk_ids", "topk_w", "counts", "offsets", "sorted_pairs", "inv")


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ROUTING_FIELDS]


# name -> (restype, argtypes); the exported C symbols of the library
SIGNATURES = {
    "moe_query": (c_i32, [ctypes.POINTER(MoeConfig), c_i32, ctypes.POINTER(c_size), ctypes.POINTER(c_size)]),
    "moe_query_workspace_layout": (c_i32, [ctypes.POINTER(MoeConfig), c_i32, ctypes.POINTER(c_size)]),
    "moe_create": (c_i32, [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights), c_vp, c_size, c_vp,
                           ctypes.POINTER(c_vp)]),
    "moe_route": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, ctypes.POINTER(MoeRouting), c_vp, c_size, c_vp]),
    "moe_forward": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(MoeRouting), c_vp, c_vp, c_size, c_vp]),
    "moe_route_forward": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, ctypes.POINTER(MoeRouting), c_vp, c_vp, c_size,
                                  c_vp]),
    "moe_route_forward_static": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, ctypes.POINTER(MoeRouting), c_vp, c_vp]),
    "moe_graph_create": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, ctypes.POINTER(MoeRouting), c_vp, c_vp, c_size,
                                 ctypes.POINTER(c_vp)]),
    "moe_graph_launch": (c_i32, [c_vp, c_vp]),
    "moe_graph_destroy": (None, [c_vp]),
    "moe_unpack_expert": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "moe_profile_begin": (c_i32, [c_vp, c_i32]),
    "moe_profile_end": (c_i32, [c_vp, ctypes.POINTER(c_i32), ctypes.POINTER(ctypes.c_float), ctypes.POINTER(c_i32)]),
    "moe_destroy": (None, [c_vp]),
    "moe_strerror": (ctypes.c_char_p, [c_i32]),
}

_lib = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run mxfp4_latent_mixture_sigmoid_amd.build.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().moe_strerror(status).decode()
        super().__init__(f"{where}: {Status(status).name if status in Status._value2member_map_ else status} ({msg})")


def check(status: int, where: str) -> None:
    if status != Status.OK:
        raise MoEError(status, where)


def ptr(t) -> int | None:
    """Device (or host) address of a tensor, None for None."""
    return None if t is None else t.data_ptr()


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_vp(s.cuda_stream)


def make_config(hidden, latent, n_experts, top_k, inter, n_shared, shared_inter, has_latent_proj,
                stage2_fp8: bool = False, stage1_a4: bool = False, shared_stream: bool = False) -> MoeConfig:
    return MoeConfig(hidden, latent, n_experts, top_k, inter, n_shared, shared_inter,
                     int(bool(has_latent_proj)), ACT_SILU_GLU, STAGE2_FP8 if stage2_fp8 else STAGE2_BF16,
                     STAGE1_MXFP4 if stage1_a4 else STAGE1_BF16, SHARED_STREAM if shared_stream else SHARED_FUSED)


def query(cfg: MoeConfig, T_max: int):
    pb, wb = c_size(0), c_size(0)
    check(lib().moe_query(ctypes.byref(cfg), T_max, ctypes.byref(pb), ctypes.byref(wb)), "moe_query")
    return pb.value, wb.value


WS_REGIONS = ("logits", "hist", "tiles", "z", "acat", "h", "y", "h8", "z4", "partials", "total")


def workspace_layout(cfg: MoeConfig, T: int) -> dict:
    arr = (c_size * len(WS_REGIONS))()
    check(lib().moe_query_workspace_layout(ctypes.byref(cfg), T, arr), "moe_query_workspace_layout")
    return dict(zip(WS_REGIONS, list(arr)))


def create(cfg: MoeConfig, weights: dict, packed, stream=None) -> c_vp:
    w = MoeWeights(*[ptr(weights.get(n)) for n in WEIGHT_FIELDS])
    h = c_vp()
    check(lib().moe_create(ctypes.byref(cfg), ctypes.byref(w), ptr(packed), packed.numel(),
                           stream_handle(stream), ctypes.byref(h)), "moe_create")
    return h


def routing_struct(r: dict) -> MoeRouting:
    return MoeRouting(*[ptr(r[n]) for n in ROUTING_FIELDS])


def route(h, x, T, routing: dict, workspace, logit_bias=None, logits_in=None, logits_out=None,
          stream=None) -> None:
    rs = routing_struct(routing)
    check(lib().moe_route(h, ptr(x), T, ptr(logit_bias), ptr(logits_in), ptr(logits_out), ctypes.byref(rs),
                          ptr(workspace), workspace.numel(), stream_handle(stream)), "moe_route")


def forward(h, x, T, routing: dict, out, workspace, stream=None) -> None:
    rs = routing_struct(routing)
    check(lib().moe_forward(h, ptr(x), T, ctypes.byref(rs), ptr(out), ptr(workspace), workspace.numel(),
                            stream_handle(stream)), "moe_forward")


def route_forward(h, x, T, routing: dict, out, workspace, logit_bias=None, logits_out=None, stream=None) -> None:
    rs = routing_struct(routing)
    check(lib().moe_route_forward(h, ptr(x), T, ptr(logit_bias), ptr(logits_out), ctypes.byref(rs), ptr(out),
                                  ptr(workspace), workspace.numel(), stream_handle(stream)), "moe_route_forward")


STATIC_SCRATCH_BYTES = 40 << 20   # MOE_STATIC_SCRATCH_BYTES


def route_forward_static(h, x, T, routing: dict, out, logit_bias=None, logits_out=None, stream=None) -> None:
    """moe_route_forward_static: no workspace argument (the library's per-GPU scratch array)."""
    rs = routing_struct(routing)
    check(lib().moe_route_forward_static(h, ptr(x), T, ptr(logit_bias), ptr(logits_out), ctypes.byref(rs), ptr(out),
                                         stream_handle(stream)), "moe_route_forward_static")


def graph_create(h, x, T, routing: dict, out, workspace, logit_bias=None, logits_out=None):
    """moe_graph_create: moe_route_forward captured for these buffers; returns the graph handle."""
    rs = routing_struct(routing)
    g = c_vp()
    check(lib().moe_graph_create(h, ptr(x), T, ptr(logit_bias), ptr(logits_out), ctypes.byref(rs), ptr(out),
                                 ptr(workspace), workspace.numel(), ctypes.byref(g)), "moe_graph_create")
    return g


def graph_launch(g, stream=None) -> None:
    check(lib().moe_graph_launch(g, stream_handle(stream)), "moe_graph_launch")


def graph_destroy(g) -> None:
    lib().moe_graph_destroy(g)


def unpack_expert(h, e: int, which: int, out, stream=None) -> None:
    check(lib().moe_unpack_expert(h, e, which, ptr(out), stream_handle(stream)), "moe_unpack_expert")


KERNELS = ("router", "topk", "permute", "xside", "tilemap", "gateup", "down", "combine", "out", "xside_epi",
           "out_epi", "router_xside", "h_quant", "z_quant", "shared")


def profile_begin(h, max_launches: int) -> None:
    check(lib().moe_profile_begin(h, max_launches), "moe_profile_begin")


def profile_end(h, max_launches: int) -> list:
    """[(kernel name, elapsed ms)] for every launch recorded since profile_begin."""
    ids = (c_i32 * max_launches)()
    ms = (ctypes.c_float * max_launches)()
    n = c_i32(max_launches)
    check(lib().moe_profile_end(h, ids, ms, ctypes.byref(n)), "moe_profile_end")
    return [(KERNELS[ids[i]], float(ms[i])) for i in range(n.value)]


def destroy(h) -> None:
    lib().moe_destroy(h)
