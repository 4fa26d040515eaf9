"""Pins for the oracle's latent projections, routed GLU experts, combine and shared experts."""
from dataclasses import replace

import numpy as np
import scipy.special

from oracle import oracle as O
from tests import _np_ref as R
from workload import SHAPES, make_inputs


def _f64(bits):
    return R.bf16_bits_to_f64(bits)


def _close_bf16(a, b, frac=2e-3):
    """Equal BF16 arrays up to rare one-ulp flips (summation order differs between the oracle's
    index loops and BLAS)."""
    a = np.asarray(a, np.uint16).astype(np.int32)
    b = np.asarray(b, np.uint16).astype(np.int32)
    diff = a != b
    assert diff.mean() <= frac, diff.mean()
    assert np.all(np.abs(a[diff] - b[diff]) <= 1)


def test_latent_down_and_output_vs_matmul():
    s = SHAPES["tiny"]
    inp = make_inputs(s, ["x", "w_down", "w_up"])
    z = O.latent_down(inp["x"], inp["w_down"])
    _close_bf16(z, R.bf16_rne(_f64(inp["x"]) @ _f64(inp["w_down"]).T))
    ys = np.random.default_rng(1).standard_normal((s.T, s.H))
    out = O.output(z, inp["w_up"], ys)
    _close_bf16(out, R.bf16_rne(_f64(z) @ _f64(inp["w_up"]).T + ys))
    out0 = O.output(z, inp["w_up"], None)
    _close_bf16(out0, R.bf16_rne(_f64(z) @ _f64(inp["w_up"]).T))


def test_shared_vs_numpy_glu():
    s = replace(SHAPES["tiny"], S=2, T=16)
    inp = make_inputs(s, ["x", "sh_gate", "sh_up", "sh_down"])
    hs, ys = O.shared(inp["x"], inp["sh_gate"], inp["sh_up"], inp["sh_down"])
    x = _f64(inp["x"])
    ref_y = np.zeros((s.T, s.H))
    for j in range(s.S):
        g = x @ _f64(inp["sh_gate"][j]).T
        u = x @ _f64(inp["sh_up"][j]).T
        h = R.bf16_rne(g * scipy.special.expit(g) * u)
        _close_bf16(hs[:, j * s.Is:(j + 1) * s.Is], h)
        ref_y += _f64(h) @ _f64(inp["sh_down"][j]).T
    assert np.allclose(ys, ref_y, rtol=1e-6, atol=1e-6)


def test_experts_single_expert_is_dense_glu_mlp():
    # E = K = 1: every token goes to expert 0 with gate weight exactly 1, so the routed layer is
    # a dense GLU MLP on the latent.
    s = replace(SHAPES["tiny"], E=1, K=1, T=24)
    inp = make_inputs(s)
    r = O.forward(inp, K=1)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    wg = R.dequant_table(inp["gate_codes"][0], inp["gate_scales"][0])
    wu = R.dequant_table(inp["up_codes"][0], inp["up_scales"][0])
    wd = R.dequant_table(inp["down_codes"][0], inp["down_scales"][0])
    h, y = R.glu_mlp(_f64(r["z"]), wg, wu, wd)
    _close_bf16(r["h"], h)
    _close_bf16(r["zc"], y, frac=5e-3)


def test_gather_equals_dense_masked_formulation():
    s = replace(SHAPES["tiny"], T=24)
    inp = make_inputs(s)
    r = O.forward(inp, K=s.K)
    ids, zc = R.masked_moe(r["z"], inp, r["logits"], s.K)
    assert np.array_equal(ids, r["ids"])
    _close_bf16(r["zc"], zc, frac=5e-3)


def test_token_permutation_invariance_bitwise():
    s = replace(SHAPES["tiny"], T=20)
    inp = make_inputs(s)
    r = O.forward(inp, K=s.K)
    perm = np.random.default_rng(9).permutation(s.T)
    inp2 = dict(inp, x=inp["x"][perm])
    r2 = O.forward(inp2, K=s.K)
    assert np.array_equal(r2["out"], r["out"][perm])
    assert np.array_equal(r2["ids"], r["ids"][perm])


def test_expert_relabelling_invariance():
    s = replace(SHAPES["tiny"], T=20, E=12, K=3)
    inp = make_inputs(s)
    r = O.forward(inp, K=s.K)
    pi = np.random.default_rng(10).permutation(s.E)      # new expert j is old expert pi[j]
    inp2 = dict(inp)
    for k in ("w_router", "gate_codes", "gate_scales", "up_codes", "up_scales",
              "down_codes", "down_scales"):
        inp2[k] = inp[k][pi]
    r2 = O.forward(inp2, K=s.K)
    assert np.array_equal(pi[r2["ids"]], r["ids"])
    assert np.array_equal(r2["out"], r["out"])


def test_power_of_two_scale_equivariance():
    # Raising every down-projection scale by one doubles every y exactly; with no shared expert
    # the combine and the up-projection are linear, so the output doubles exactly.
    s = replace(SHAPES["tiny"], T=16, S=0)
    inp = make_inputs(s)
    r = O.forward(inp, K=s.K)
    inp2 = dict(inp, down_scales=(inp["down_scales"] + 1).astype(np.uint8))
    r2 = O.forward(inp2, K=s.K)
    assert np.array_equal(_f64(r2["y"]), 2 * _f64(r["y"]))
    assert np.array_equal(_f64(r2["out"]), 2 * _f64(r["out"]))


def test_unit_scales_integer_exact():
    # With all scales 127 and small integer-valued latents every expert product is a sum of
    # half-integers: the oracle's g and u equal the exact integer arithmetic.
    s = replace(SHAPES["tiny"], T=4, E=2, K=1, Lt=64, I=32)
    inp = make_inputs(s, ["gate_codes", "up_codes", "down_codes"])
    for m in ("gate", "up", "down"):
        inp[m + "_scales"] = np.full(inp[m + "_codes"].shape[:2] + (inp[m + "_codes"].shape[2] // 16,),
                                     127, np.uint8)
    z = R.bf16_rne(np.random.default_rng(2).integers(-1, 2, (s.T, s.Lt)) / 16.0)
    ids = np.zeros((s.T, 1), np.int32)
    h, y = O.experts(z, ids, inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                     inp["up_scales"], inp["down_codes"], inp["down_scales"])
    zi = (_f64(z) * 16).astype(np.int64)                 # 16 z is an integer
    gc = (R.dequant_table(inp["gate_codes"][0], inp["gate_scales"][0]) * 2).astype(np.int64)
    uc = (R.dequant_table(inp["up_codes"][0], inp["up_scales"][0]) * 2).astype(np.int64)
    g = (zi @ gc.T) / 32.0
    u = (zi @ uc.T) / 32.0
    _close_bf16(h, R.bf16_rne(g * scipy.special.expit(g) * u))


def test_split_halves_equal_whole_steps():
    # The down halves evaluated on the whole steps' own intermediates reproduce them bitwise.
    s = replace(SHAPES["tiny"], T=12, S=2)
    inp = make_inputs(s)
    r = O.forward(inp, K=s.K)
    y = O.expert_down(r["h"], r["ids"], inp["down_codes"], inp["down_scales"])
    assert np.array_equal(y, r["y"])
    ys = O.shared_down(r["hs"], inp["sh_down"])
    assert np.array_equal(ys, r["ys"])
