"""GPU parity: the HIP path (through the C ABI) against the FP64 CPU oracle.

Routing ids and the expert grouping must match bit for bit (the oracle selects on the GPU's own
FP32 logits); every floating-point tensor (logits, z, h, y, zc, h_s, out) must satisfy
max|err| <= 2e-2 rms(ref) and mean|err| <= 2e-3 rms(ref); gate weights match to 1e-6 relative.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_helpers as G
from workload import SHAPES, LayerShape, make_inputs, sample_tokens, tie_tokens

pytestmark = pytest.mark.gpu

MID = LayerShape("mid", 200, 1024, 512, 64, 8, 256, 2, 128, True, "uniform", 0.0, 7)
MID_ZIPF = LayerShape("mid_zipf", 300, 1024, 512, 96, 6, 256, 1, 256, True, "zipf", 0.0, 8)
NOLAT = LayerShape("nolat", 77, 512, 512, 32, 4, 256, 0, 0, False, "uniform", 0.0, 9)
# Many rows per expert (300 * 4 / 16 = 75 on average, Zipf-skewed): the matrix-core tiled path for
# the dense and the grouped products, with ragged row tiles and empty experts.
PREFILL_SMALL = LayerShape("prefill_small", 300, 1024, 512, 16, 4, 256, 1, 128, True, "zipf", 0.0, 12)
NOLAT_TILED = LayerShape("nolat_tiled", 260, 384, 384, 8, 3, 384, 0, 0, False, "uniform", 0.0, 13)
# Many rows per expert at 2I = 768 (three 256-column tiles per row tile on the tiled kernel),
# Zipf-skewed, with ragged prefixes.
PREFILL_GLU = LayerShape("prefill_glu", 300, 1024, 512, 16, 4, 384, 1, 128, True, "zipf", 0.0, 15)
# One or two rows per expert (24 * 4 / 128 < 1): the decode expert kernels with 4-row tiles and the
# activations staged in LDS.
SPARSE = LayerShape("sparse", 24, 1024, 512, 128, 4, 256, 1, 128, True, "uniform", 0.0, 14)
SMALL_SHAPES = {s.name: s for s in (SHAPES["tiny"], MID, MID_ZIPF, NOLAT, PREFILL_SMALL, NOLAT_TILED, SPARSE,
                                     PREFILL_GLU)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


_cache = {}


def _setup(name):
    if name not in _cache:
        shape = SMALL_SHAPES[name]
        G.log(f"[setup] {name}: T={shape.T} E={shape.E} K={shape.K}")
        inp = make_inputs(shape)
        layer = G.make_layer(shape, inp, T_max=shape.T)
        _cache[name] = (shape, inp, layer)
    return _cache[name]


@pytest.mark.parametrize("name", list(SMALL_SHAPES))
def test_unpack_bit_exact(name):
    shape, inp, layer = _setup(name)
    for e in sorted({0, shape.E // 2, shape.E - 1}):
        for which, (c, s) in enumerate((("gate_codes", "gate_scales"), ("up_codes", "up_scales"),
                                        ("down_codes", "down_scales"))):
            got = G.host_bf16(layer.unpack_expert(e, which))
            ref = O.f64_to_bf16(O.dequant(inp[c][e], inp[s][e]))
            assert np.array_equal(got, ref), (name, e, which)


def test_unpack_scale_range_bit_exact():
    # Every E8M0 byte whose products stay in BF16's normal range converts exactly.
    shape = replace(SHAPES["tiny"], E=2, name="scales")
    inp = make_inputs(shape)
    rng = np.random.default_rng(1)
    for m in ("gate", "up", "down"):
        inp[m + "_scales"] = rng.integers(2, 253, inp[m + "_scales"].shape).astype(np.uint8)
    layer = G.make_layer(shape, inp, T_max=1)
    for which, (c, s) in enumerate((("gate_codes", "gate_scales"), ("up_codes", "up_scales"),
                                    ("down_codes", "down_scales"))):
        got = G.host_bf16(layer.unpack_expert(1, which))
        ref = O.f64_to_bf16(O.dequant(inp[c][1], inp[s][1]))
        assert np.array_equal(got, ref)


def test_unpack_special_scales():
    """E8M0 bytes 0 and 1 (products down to BF16 subnormals, 2^-128), 2 and 255 (NaN for every code of
    the block): exact bits where the oracle's value is a number, NaN where it is NaN."""
    shape = replace(SHAPES["tiny"], E=2, name="scales")
    inp = make_inputs(shape)
    rng = np.random.default_rng(2)
    for m in ("gate", "up", "down"):
        inp[m + "_scales"] = rng.choice(np.array([0, 1, 2, 255], np.uint8), inp[m + "_scales"].shape)
    layer = G.make_layer(shape, inp, T_max=1)
    for which, (c, s) in enumerate((("gate_codes", "gate_scales"), ("up_codes", "up_scales"),
                                    ("down_codes", "down_scales"))):
        got = G.host_bf16(layer.unpack_expert(1, which))
        refv = O.dequant(inp[c][1], inp[s][1])
        nan = np.isnan(refv)
        assert nan.any() and (~nan).any()
        gotv = G.bf16_f64(got)
        assert np.all(np.isnan(gotv[nan])), which
        assert np.array_equal(got[~nan], O.f64_to_bf16(refv)[~nan]), which


@pytest.mark.parametrize("name", list(SMALL_SHAPES))
def test_forward_parity(name):
    shape, inp, layer = _setup(name)
    G.log(f"[forward] {name}")
    run = G.GpuRun(layer, shape, inp)
    G.check_forward(shape, inp, run)
    if shape.routing == "zipf" and shape.E >= 64:
        assert np.sum(run.counts == 0) > 0, "skewed routing over many experts should leave some empty"


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_deterministic_and_token_permutation_invariant(name):
    shape, inp, layer = _setup(name)
    a = G.GpuRun(layer, shape, inp)
    b = G.GpuRun(layer, shape, inp)
    ra, rb = a.rows(), b.rows()
    assert np.array_equal(ra["out"], rb["out"]) and np.array_equal(a.ids, b.ids)
    assert np.array_equal(ra["y"], rb["y"]) and np.array_equal(ra["h"], rb["h"])
    perm = np.random.default_rng(3).permutation(shape.T)
    c = G.GpuRun(layer, shape, dict(inp, x=inp["x"][perm]))
    assert np.array_equal(c.ids, a.ids[perm])
    assert np.array_equal(c.rows()["out"], ra["out"][perm])


@pytest.mark.parametrize("T", [1, 2, 15, 17, 33])
def test_ragged_token_counts(T):
    shape, inp, layer = _setup("mid")
    sub = dict(inp, x=inp["x"][:T])
    run = G.GpuRun(layer, shape, sub)
    G.check_forward(replace(shape, T=T), sub, run)


@pytest.mark.parametrize("T", [257, 283])
def test_tiled_expert_paths_768_ragged(T):
    """Prefixes of prefill_glu (2I = 768) on the tiled expert path, every token compared."""
    shape, inp, layer = _setup("prefill_glu")
    sub = dict(inp, x=inp["x"][:T])
    run = G.GpuRun(layer, shape, sub)
    G.check_forward(replace(shape, T=T), sub, run)


@pytest.mark.parametrize("T", [128, 131, 257])
def test_tiled_expert_paths_ragged(T):
    """Prefixes of prefill_small on the tiled expert path: partial tiles of every fragment count
    (the 3-, 4-, 5- and 6-fragment code paths among them), every token compared."""
    shape, inp, layer = _setup("prefill_small")
    sub = dict(inp, x=inp["x"][:T])
    run = G.GpuRun(layer, shape, sub)
    G.check_forward(replace(shape, T=T), sub, run)


@pytest.mark.parametrize("name", list(SMALL_SHAPES))
def test_route_forward_bit_identical(name):
    shape, inp, layer = _setup(name)
    run = G.GpuRun(layer, shape, inp)
    G.check_fused_identical(layer, shape, inp, run)


@pytest.mark.parametrize("T", [1, 17, 64, 65])
def test_route_forward_ragged_and_size_boundaries(T):
    """Around the few-token paths: T = 64 is the last split-K size, 65 the first tiled one."""
    shape = replace(MID, name=f"fused{T}", T=T, seed=21)
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=shape.T)
    run = G.GpuRun(layer, shape, inp)
    G.check_fused_identical(layer, shape, inp, run)
    G.check_forward(shape, inp, run)
    layer.close()


def test_route_forward_zero_tokens_and_bad_arguments():
    from mxfp4_latent_mixture_sigmoid_amd import abi
    shape, inp, layer = _setup("tiny")
    x = G.dev(inp["x"])
    r = layer.alloc_routing(1)
    r["counts"].fill_(-7)
    out = torch.full((1, shape.H), 3.0, dtype=torch.bfloat16, device="cuda")
    abi.route_forward(layer.handle, x, 0, r, out, layer.workspace)
    torch.cuda.synchronize()
    assert int(r["counts"][0]) == -7 and float(out[0, 0]) == 3.0
    r = layer.alloc_routing(shape.T)
    out = torch.empty(shape.T, shape.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(abi.MoEError) as ei:       # workspace too small
        abi.route_forward(layer.handle, x, shape.T, r, out, layer.workspace[:256])
    assert ei.value.status == abi.Status.BUFFER_TOO_SMALL
    with pytest.raises(abi.MoEError) as ei:       # output aliases input
        abi.route_forward(layer.handle, x, shape.T, r, x, layer.workspace)
    assert ei.value.status == abi.Status.INVALID_ARG
    lg = torch.empty(shape.T, shape.E, dtype=torch.float32, device="cuda")
    with pytest.raises(abi.MoEError) as ei:       # logits_out aliases the output
        abi.route_forward(layer.handle, x, shape.T, r, out, layer.workspace, logits_out=out)
    assert ei.value.status == abi.Status.INVALID_ARG


def test_zero_tokens_is_noop():
    shape, inp, layer = _setup("tiny")
    r = layer.alloc_routing(1)
    r["counts"].fill_(-7)
    layer.route(G.dev(inp["x"]), 0, r)
    out = torch.full((1, shape.H), 3.0, dtype=torch.bfloat16, device="cuda")
    layer.forward(G.dev(inp["x"]), 0, r, out=out)
    torch.cuda.synchronize()
    assert int(r["counts"][0]) == -7 and float(out[0, 0]) == 3.0


@pytest.mark.parametrize("E,K", [(16, 16), (48, 1), (8, 8)])
def test_degenerate_topk(E, K):
    shape = replace(MID, name=f"deg{E}_{K}", T=40, E=E, K=K, seed=11)
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=shape.T)
    run = G.GpuRun(layer, shape, inp)
    G.check_forward(shape, inp, run)
    if K == E:
        assert np.all(np.sort(run.ids, 1) == np.arange(E))
    if K == 1:
        assert np.all(run.w == 1.0)


def test_planted_ties_select_lower_index():
    shape, inp, layer = _setup("mid")
    run = G.GpuRun(layer, shape, inp)
    lg = run.logits.copy()
    toks = np.arange(0, shape.T, 7)
    order = O.select(lg[toks].astype(np.float64), shape.K + 1)
    e_k, e_k1 = order[:, shape.K - 1], order[:, shape.K]
    lg[toks, e_k1] = lg[toks, e_k]
    tied = G.GpuRun(layer, shape, dict(inp), logits_in=lg)
    lo = np.minimum(e_k, e_k1)
    hi = np.maximum(e_k, e_k1)
    assert all(lo[i] in tied.ids[t] and hi[i] not in tied.ids[t] for i, t in enumerate(toks))
    G.check_forward(shape, inp, tied, oracle_logits_in=lg)


@pytest.mark.parametrize("grid", [4.0, 0.25])
def test_heavy_ties_select_lower_index(grid):
    """Logits rounded to a coarse grid tie most of the 96 experts: with grid 4 nearly all of them
    share the top value (more than 64 candidates for the last places), with 0.25 a few do. Either
    way the selection must equal the oracle's (logit descending, lower expert first), bit for bit."""
    shape, inp, layer = _setup("mid_zipf")
    run = G.GpuRun(layer, shape, inp)
    lg = (np.round(run.logits / grid) * grid).astype(np.float32)
    top = np.sort(lg, 1)[:, ::-1]
    assert np.any(top[:, shape.K - 1] == top[:, shape.K])        # ties straddle rank K
    tied = G.GpuRun(layer, shape, dict(inp), logits_in=lg)
    G.check_forward(shape, inp, tied, oracle_logits_in=lg)


def test_power_of_two_down_scales_double_the_output_bitwise():
    """Raising every down-matrix E8M0 scale by one doubles each expert output exactly; with the
    shared experts zeroed, zc and the output then double bit for bit too (every step is a product
    or an FP32 sum of doubled terms, and BF16 rounding commutes with doubling). Routing is
    untouched."""
    shape = replace(MID, name="pow2", seed=23)
    inp = make_inputs(shape)
    inp0 = dict(inp, **{k: np.zeros_like(inp[k]) for k in ("sh_gate", "sh_up", "sh_down")})
    inp1 = dict(inp0, down_scales=(inp0["down_scales"] + 1).astype(np.uint8))
    runs = []
    for d in (inp0, inp1):
        layer = G.make_layer(shape, d, T_max=shape.T)
        run = G.GpuRun(layer, shape, d)
        runs.append((run, run.rows()))
        layer.close()
    (a, ra), (b, rb) = runs
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.w, b.w)
    for k in ("y", "zc", "out"):
        assert np.array_equal(G.bf16_f64(rb[k]), 2.0 * G.bf16_f64(ra[k])), k
    assert np.any(G.bf16_f64(ra["out"]) != 0.0)


def test_expert_relabelling_leaves_the_output_unchanged_bitwise():
    """Relabelling the experts consistently (router rows and every expert matrix moved to the new
    index) selects the relabelled experts in the same rank order with the same weights, and every
    expert row is computed from the same data in the same order: the output is bit-identical."""
    shape = replace(MID, name="relabel", seed=29)
    inp = make_inputs(shape)
    perm = np.random.default_rng(5).permutation(shape.E)     # expert e becomes perm[e]
    moved = dict(inp)
    for k in ("w_router", "gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales"):
        a = np.empty_like(inp[k])
        a[perm] = inp[k]
        moved[k] = a
    if inp.get("router_bias") is not None:
        b = np.empty_like(inp["router_bias"])
        b[perm] = inp["router_bias"]
        moved["router_bias"] = b
    runs = []
    for d in (inp, moved):
        layer = G.make_layer(shape, d, T_max=shape.T)
        run = G.GpuRun(layer, shape, d)
        runs.append((run, run.rows()))
        layer.close()
    (a, ra), (b, rb) = runs
    assert np.array_equal(b.ids, perm[a.ids]) and np.array_equal(a.w, b.w)
    for k in ("z", "y", "zc", "hs", "out"):
        assert np.array_equal(ra[k], rb[k]), k


def test_bad_arguments_raise():
    from mxfp4_latent_mixture_sigmoid_amd import abi
    shape, inp, layer = _setup("tiny")
    r = layer.alloc_routing(shape.T)
    x = G.dev(inp["x"])
    with pytest.raises(abi.MoEError) as ei:       # logits_in together with x
        abi.route(layer.handle, x, shape.T, r, layer.workspace, logits_in=torch.zeros(1, device="cuda"))
    assert ei.value.status == abi.Status.INVALID_ARG
    with pytest.raises(abi.MoEError) as ei:       # workspace too small
        abi.route(layer.handle, x, shape.T, r, layer.workspace[:256])
    assert ei.value.status == abi.Status.BUFFER_TOO_SMALL
    with pytest.raises(abi.MoEError):             # output aliases input
        abi.forward(layer.handle, x, shape.T, r, x, layer.workspace)
