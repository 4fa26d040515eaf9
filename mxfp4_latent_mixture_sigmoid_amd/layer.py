"""MoELayer: owns the packed weights, workspace and routing buffers of one layer on one GPU and
calls the C ABI (torch provides device memory and the stream; all arithmetic runs in HIP)."""
from __future__ import annotations

import torch

from . import abi


class MoELayer:
    """One MXFP4 latent-MoE layer on the current GPU.

    ``weights`` maps the canonical weight names of ``abi.WEIGHT_FIELDS`` to device tensors
    (BF16 bit patterns as int16/bfloat16, MXFP4 codes/scales as uint8); they are only read while
    the packing kernels run and may be dropped after the first synchronisation.

    ``stage2_fp8`` quantises h to MX FP8 for the down product (MOE_STAGE2_FP8); ``stage1_a4``
    quantises z to MX FP4 for the gate/up product (MOE_STAGE1_MXFP4, A4W4). Both default to the
    BF16 layer; each adds one packed copy of the weights it changes. ``shared_stream`` runs the
    shared experts' gate/up product on a second stream owned by the handle, concurrently with the
    routing and the routed experts (MOE_SHARED_STREAM); the outputs are the same bits.
    """

    def __init__(self, hidden, latent, n_experts, top_k, inter, n_shared, shared_inter,
                 has_latent_proj, weights: dict, T_max: int, device="cuda", stream=None,
                 stage2_fp8: bool = False, stage1_a4: bool = False, shared_stream: bool = False):
        self.cfg = abi.make_config(hidden, latent, n_experts, top_k, inter, n_shared, shared_inter,
                                   has_latent_proj, stage2_fp8, stage1_a4, shared_stream)
        self.E, self.K, self.Lt = n_experts, top_k, latent
        self.H = hidden if has_latent_proj else latent
        self.T_max = T_max
        packed_bytes, ws_bytes = abi.query(self.cfg, T_max)
        self.device = torch.device(device)
        self.packed = torch.empty(packed_bytes, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.handle = abi.create(self.cfg, weights, self.packed, stream)

    def alloc_routing(self, T: int) -> dict:
        d, P = self.device, max(T * self.K, 1)
        i32 = dict(dtype=torch.int32, device=d)
        return dict(topk_ids=torch.empty(max(T, 1), self.K, **i32),
                    topk_w=torch.empty(max(T, 1), self.K, dtype=torch.float32, device=d),
                    counts=torch.empty(self.E, **i32), offsets=torch.empty(self.E + 1, **i32),
                    sorted_pairs=torch.empty(P, **i32), inv=torch.empty(P, **i32))

    def _check_T(self, T):
        if T > self.T_max:
            raise ValueError(f"T={T} exceeds T_max={self.T_max}")

    def route(self, x, T, routing, logit_bias=None, logits_in=None, logits_out=None, stream=None):
        self._check_T(T)
        abi.route(self.handle, x, T, routing, self.workspace, logit_bias, logits_in, logits_out, stream)

    def forward(self, x, T, routing, out=None, stream=None):
        self._check_T(T)
        if out is None:
            out = torch.empty(max(T, 1), self.H, dtype=torch.bfloat16, device=self.device)
        abi.forward(self.handle, x, T, routing, out, self.workspace, stream)
        return out

    def route_forward(self, x, T, routing, out=None, logit_bias=None, logits_out=None, stream=None):
        """route + forward in one call, bitwise identical to the two calls."""
        self._check_T(T)
        if out is None:
            out = torch.empty(max(T, 1), self.H, dtype=torch.bfloat16, device=self.device)
        abi.route_forward(self.handle, x, T, routing, out, self.workspace, logit_bias, logits_out, stream)
        return out

    def route_forward_static(self, x, T, routing, out=None, logit_bias=None, logits_out=None, stream=None):
        """route + forward in the library's per-GPU scratch array instead of this layer's workspace
        (the call allocates nothing; bitwise identical to route_forward)."""
        if out is None:
            out = torch.empty(max(T, 1), self.H, dtype=torch.bfloat16, device=self.device)
        abi.route_forward_static(self.handle, x, T, routing, out, logit_bias, logits_out, stream)
        return out

    def graph(self, x, T, routing, out, logit_bias=None, logits_out=None):
        """route_forward captured as one HIP graph on these buffers (see StepGraph)."""
        self._check_T(T)
        return StepGraph(self, abi.graph_create(self.handle, x, T, routing, out, self.workspace, logit_bias,
                                                logits_out), (x, routing, out, logit_bias, logits_out))

    def unpack_expert(self, e: int, which: int, stream=None):
        rows, cols = (self.cfg.inter, self.Lt) if which < 2 else (self.Lt, self.cfg.inter)
        out = torch.empty(rows, cols, dtype=torch.bfloat16, device=self.device)
        abi.unpack_expert(self.handle, e, which, out, stream)
        return out

    def workspace_view(self, T: int, region: str, shape, dtype):
        """Tensor view of a workspace region (test hook)."""
        off = abi.workspace_layout(self.cfg, T)[region]
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)

    def close(self):
        if self.handle:
            abi.destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepGraph:
    """One captured route_forward: launch() replays it on the buffers it was captured with (write
    each step's tokens into the same x tensor). Holds references to those buffers and the layer."""

    def __init__(self, layer, g, buffers):
        self.layer, self.g, self.buffers = layer, g, buffers

    def launch(self, stream=None):
        if not self.g:
            raise RuntimeError("graph destroyed")
        abi.graph_launch(self.g, stream)

    def close(self):
        if self.g:
            abi.graph_destroy(self.g)
            self.g = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
