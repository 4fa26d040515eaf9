"""GPU: the shared experts' gate/up product on the handle's second stream (MOE_SHARED_STREAM).

The mode only moves where h_s is computed: every output must equal the fused mode's (whose outputs
the parity tests hold to the FP64 oracle) bit for bit -- routing arrays, logits and output, through
moe_route_forward, moe_route + moe_forward and moe_route_forward_static, on the few-token
(split-K) and the many-token paths -- and a HIP graph captured with the fork and join must replay to the same bits."""
from dataclasses import replace

import pytest
import torch

from tests import gpu_helpers as G
from workload import SHAPES, LayerShape, make_inputs

pytestmark = pytest.mark.gpu

MID = LayerShape("mid", 200, 1024, 512, 64, 8, 256, 2, 128, True, "uniform", 0.0, 7)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


def _run(layer, shape, inp, x, T, bias, two_calls):
    r = layer.alloc_routing(T)
    lg = torch.empty(T, shape.E, dtype=torch.float32, device="cuda")
    if two_calls:
        layer.route(x, T, r, logit_bias=bias, logits_out=lg)
        out = layer.forward(x, T, r)
    else:
        out = layer.route_forward(x, T, r, logit_bias=bias, logits_out=lg)
    torch.cuda.synchronize()
    return r, lg, out


def _same(tag, a, b, T, K):
    (r, lg, out), (r2, lg2, out2) = a, b
    for k in ("topk_ids", "counts", "offsets"):
        assert torch.equal(r[k], r2[k]), f"{tag}: {k}"
    assert torch.equal(r["topk_w"].view(torch.int32), r2["topk_w"].view(torch.int32)), f"{tag}: topk_w"
    for k in ("sorted_pairs", "inv"):
        assert torch.equal(r[k][:T * K], r2[k][:T * K]), f"{tag}: {k}"
    assert torch.equal(lg.view(torch.int32), lg2.view(torch.int32)), f"{tag}: logits"
    assert torch.equal(out[:T].view(torch.int16), out2[:T].view(torch.int16)), f"{tag}: output"


def _check(shape, T, graph=False):
    G.log(f"[shared-stream] {shape.name} T={T} graph={graph}")
    inp = make_inputs(replace(shape, T=T))
    fused = G.make_layer(shape, inp, T_max=T)
    apart = G.make_layer(shape, inp, T_max=T, shared_stream=True)
    bias = None if inp.get("router_bias") is None else G.dev(inp["router_bias"])
    x = G.dev(inp["x"])
    try:
        for two in (False, True):
            ref = _run(fused, shape, inp, x, T, bias, two)
            got = _run(apart, shape, inp, x, T, bias, two)
            _same(f"{shape.name} T={T} {'route+forward' if two else 'route_forward'}", ref, got, T, shape.K)
        if T <= 64:   # the allocation-free entry point: the second stream's partials in the scratch array
            ref = _run(fused, shape, inp, x, T, bias, False)
            r = apart.alloc_routing(T)
            lg = torch.empty(T, shape.E, dtype=torch.float32, device="cuda")
            out = apart.route_forward_static(x, T, r, logit_bias=bias, logits_out=lg)
            torch.cuda.synchronize()
            _same(f"{shape.name} T={T} route_forward_static", ref, (r, lg, out), T, shape.K)
        if graph:
            ref = _run(fused, shape, inp, x, T, bias, False)
            rg = apart.alloc_routing(T)
            lgg = torch.empty(T, shape.E, dtype=torch.float32, device="cuda")
            outg = torch.empty(T, apart.H, dtype=torch.bfloat16, device="cuda")
            g = apart.graph(x, T, rg, outg, logit_bias=bias, logits_out=lgg)
            try:
                for i in range(3):
                    g.launch()
                    if i == 1:
                        g.launch()
                    torch.cuda.synchronize()
                    _same(f"{shape.name} T={T} replay {i}", ref, (rg, lgg, outg), T, shape.K)
                    _run(apart, shape, inp, x, T, bias, False)   # eager work between replays
            finally:
                g.close()
    finally:
        fused.close()
        apart.close()


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
def test_shared_stream_matches_fused(T):
    _check(MID, T, graph=T in (17, 200))


def test_shared_stream_matches_fused_decode_tp8():
    _check(SHAPES["tp8_decode_t64"], 64, graph=True)


def test_shared_stream_matches_fused_prefill_tp8():
    _check(SHAPES["tp8_prefill_t8192"], 8192)
