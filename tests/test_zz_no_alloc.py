"""moe_route_forward_static, the entry point that allocates nothing (its workspace is the library's
per-GPU scratch array): bit-for-bit the results of moe_route_forward with a caller workspace, on
two calls in a row (the second with fewer tokens, so it runs on the first call's leftovers), and a
clear error before any launch when a call's workspace exceeds the array."""
import numpy as np
import pytest
import torch

from mxfp4_latent_mixture_sigmoid_amd import abi
from tests import gpu_helpers as G
from workload import SHAPES, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


def _run(layer, shape, x, bias, T, static):
    r = layer.alloc_routing(T)
    lg = torch.empty(max(T, 1), shape.E, dtype=torch.float32, device="cuda")
    out = torch.empty(max(T, 1), layer.H, dtype=torch.bfloat16, device="cuda")
    fn = layer.route_forward_static if static else layer.route_forward
    fn(x, T, r, out=out, logit_bias=bias, logits_out=lg)
    return r, lg, out


def _same(a, b, T, K, what):
    (ra, la, oa), (rb, lb, ob) = a, b
    n = {"topk_ids": T, "topk_w": T, "counts": None, "offsets": None, "sorted_pairs": T * K, "inv": T * K}
    for k, m in n.items():
        va, vb = (ra[k], rb[k]) if m is None else (ra[k][:m], rb[k][:m])
        if va.dtype == torch.float32:
            va, vb = va.view(torch.int32), vb.view(torch.int32)
        assert torch.equal(va, vb), f"{what}: {k} differs"
    assert torch.equal(la[:T].view(torch.int32), lb[:T].view(torch.int32)), f"{what}: logits differ"
    assert torch.equal(oa[:T].view(torch.int16), ob[:T].view(torch.int16)), f"{what}: output differs"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,T2", [("tiny", 23), ("tp8_decode_t64", 40), ("tp8_prefill_t8192", 57)])
def test_static_entry_matches_workspace_entry(name, T2):
    shape = SHAPES[name]
    if name == "tp8_prefill_t8192":   # the Zipf-biased router at decode size
        shape = shape.with_tokens(64)
    T1 = shape.T
    G.log(f"[no-alloc] {shape.name}: T1={T1} then T2={T2}")
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=T1)
    x = G.dev(inp["x"])
    bias = None if inp.get("router_bias") is None else G.dev(inp["router_bias"])
    # two static calls in a row, the second smaller (it finds the first call's data in the array)
    s1 = _run(layer, shape, x, bias, T1, static=True)
    s2 = _run(layer, shape, x, bias, T2, static=True)
    torch.cuda.synchronize()
    w1 = _run(layer, shape, x, bias, T1, static=False)
    w2 = _run(layer, shape, x, bias, T2, static=False)
    torch.cuda.synchronize()
    _same(s1, w1, T1, shape.K, f"T={T1}")
    _same(s2, w2, T2, shape.K, f"T={T2}")
    # and against the oracle's routing on the smaller call (bit-exact ids and grouping)
    ids = s2[0]["topk_ids"][:T2].cpu().numpy()
    ref_ids = G.O.select(s2[1][:T2].cpu().numpy().astype(np.float64), shape.K)
    assert np.array_equal(ids, ref_ids)
    G.log("  static calls bit-identical to workspace calls")
    layer.close()


@pytest.mark.timeout(300)
def test_static_entry_rejects_oversized_calls_before_any_launch():
    shape = SHAPES["tp8_decode_t64"].with_tokens(300)
    c = abi.make_config(shape.H, shape.Lt, shape.E, shape.K, shape.I, shape.S, shape.Is, shape.has_latent)
    need = abi.workspace_layout(c, 300)["total"]
    assert need > abi.STATIC_SCRATCH_BYTES
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=300)
    x = G.dev(inp["x"])
    r = layer.alloc_routing(300)
    out = torch.full((300, layer.H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(abi.MoEError) as ei:
        layer.route_forward_static(x, 300, r, out=out)
    assert ei.value.status == abi.Status.BUFFER_TOO_SMALL
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)), "nothing may be written by a rejected call"
    # T = 0 is a valid no-op
    layer.route_forward_static(x, 0, r, out=out)
    torch.cuda.synchronize()
    layer.close()
