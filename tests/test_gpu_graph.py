"""GPU: moe_route_forward captured as one HIP graph (the fused decode step) and replayed.

Every replay must equal an eager moe_route_forward on the same input bit for bit -- routing arrays,
logits and output -- including replays after the input buffer was rewritten, with other eager work
and synchronisations between replays, and several replays of one capture in a row. Eager
route_forward itself is held to the FP64 oracle by the parity tests."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from tests import gpu_helpers as G
from workload import SHAPES, LayerShape, make_inputs

pytestmark = pytest.mark.gpu

MID = LayerShape("mid", 200, 1024, 512, 64, 8, 256, 2, 128, True, "uniform", 0.0, 7)
NOLAT = LayerShape("nolat", 77, 512, 512, 32, 4, 256, 0, 0, False, "uniform", 0.0, 9)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


def _eager(layer, shape, x, T, bias):
    r = layer.alloc_routing(T)
    lg = torch.empty(T, shape.E, dtype=torch.float32, device="cuda")
    out = layer.route_forward(x, T, r, logit_bias=bias, logits_out=lg)
    return r, lg, out


def _same(tag, r, lg, out, r2, lg2, out2, T, K):
    for k in ("topk_ids", "counts", "offsets"):
        assert torch.equal(r[k], r2[k]), f"{tag}: {k}"
    assert torch.equal(r["topk_w"].view(torch.int32), r2["topk_w"].view(torch.int32)), f"{tag}: topk_w"
    for k in ("sorted_pairs", "inv"):
        assert torch.equal(r[k][:T * K], r2[k][:T * K]), f"{tag}: {k}"
    assert torch.equal(lg.view(torch.int32), lg2.view(torch.int32)), f"{tag}: logits"
    assert torch.equal(out[:T].view(torch.int16), out2[:T].view(torch.int16)), f"{tag}: output"


def _check_replays(shape, T, replays=4, stage1_a4=False, stage2_fp8=False):
    G.log(f"[graph] {shape.name} T={T} a4={stage1_a4} fp8={stage2_fp8}")
    inp = make_inputs(replace(shape, T=T))
    layer = G.make_layer(shape, inp, T_max=T, stage1_a4=stage1_a4, stage2_fp8=stage2_fp8)
    bias = None if inp.get("router_bias") is None else G.dev(inp["router_bias"])
    xs = [G.dev(inp["x"])]
    rng = np.random.default_rng(shape.seed + 101)
    for i in range(replays - 1):   # other token sets of the same shape: permuted rows, rescaled
        perm = torch.from_numpy(rng.permutation(T)).cuda()
        xb = xs[0][perm].view(torch.bfloat16).float() * (1.0 + 0.25 * (i + 1))
        xs.append(xb.to(torch.bfloat16).view(xs[0].dtype))   # same bf16-bits dtype as the input
    xg = torch.empty_like(xs[0])
    rg = layer.alloc_routing(T)
    lgg = torch.empty(T, shape.E, dtype=torch.float32, device="cuda")
    outg = torch.empty(T, layer.H, dtype=torch.bfloat16, device="cuda")
    graph = layer.graph(xg, T, rg, outg, logit_bias=bias, logits_out=lgg)
    try:
        for i, x in enumerate(xs + xs[:1]):
            xg.copy_(x)
            graph.launch()
            if i % 2:   # two replays in a row on the same input
                graph.launch()
            torch.cuda.synchronize()
            r, lg, out = _eager(layer, shape, x, T, bias)   # eager work between replays
            torch.cuda.synchronize()
            _same(f"{shape.name} T={T} replay {i}", r, lg, out, rg, lgg, outg, T, shape.K)
    finally:
        graph.close()
        layer.close()


@pytest.mark.parametrize("T", [1, 17, 64])
def test_graph_replays_match_eager_few_tokens(T):
    _check_replays(MID, T)


def test_graph_replays_match_eager_many_tokens():
    _check_replays(MID, 200)


def test_graph_replays_match_eager_without_latent_projections():
    _check_replays(NOLAT, 40)


def test_graph_replays_match_eager_decode_full_size():
    _check_replays(SHAPES["tp8_decode_t64"], 64, replays=3)


@pytest.mark.parametrize("a4,fp8", [(True, False), (False, True), (True, True)])
def test_graph_replays_match_eager_quantised_stages(a4, fp8):
    # the quantisers and the scaled-instruction expert kernels inside the captured step
    _check_replays(MID, 64, replays=3, stage1_a4=a4, stage2_fp8=fp8)


def test_graph_rejects_profiling_and_zero_tokens():
    from mxfp4_latent_mixture_sigmoid_amd import abi
    inp = make_inputs(replace(MID, T=8))
    layer = G.make_layer(MID, inp, T_max=8)
    x = G.dev(inp["x"])
    r = layer.alloc_routing(8)
    out = torch.empty(8, layer.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        layer.graph(x, 0, r, out)
    abi.profile_begin(layer.handle, 16)
    with pytest.raises(RuntimeError):
        layer.graph(x, 8, r, out)
    abi.profile_end(layer.handle, 16)
    g = layer.graph(x, 8, r, out)
    g.close()
    g.close()
    layer.close()
