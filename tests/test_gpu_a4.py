"""GPU parity of the A4W4 first stage (MOE_STAGE1_MXFP4) against the oracle's reading of it
(oracle.c, O11: OCP MX FP4 z, one E8M0 scale per 32 values along Lt; gate/up product on the
quantised values).

The quantised z is an integer result decided from the GPU's own BF16 z, so its E2M1 codes and
E8M0 scales must equal the oracle's quantisation of that same z bit for bit. h must then match the
oracle's FP64 gate/up product on those codes (FP32 accumulation of exact products: BF16 results
equal but for rare one-ulp rounding disagreements), and the whole layer must meet the end-to-end
bar from the GPU's h on, and the oracle's fully independent A4W4 forward within the mean bar
(code differences are allowed only where the BF16 z already differs). Shapes cover 16-row
expert tiles (few rows per expert) and 128-row tiles with ragged ends, empty experts, Zipf routing,
I = 128, 256 and 384, and the layer without latent projections; one shape runs both quantised
stages together.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_helpers as G
from tests.test_gpu_parity import MID, MID_ZIPF, NOLAT, NOLAT_TILED, PREFILL_SMALL, SPARSE
from workload import SHAPES

pytestmark = pytest.mark.gpu

A4_SHAPES = {s.name: s for s in (SHAPES["tiny"], MID, MID_ZIPF, NOLAT, PREFILL_SMALL, NOLAT_TILED, SPARSE)}
# h elements bitwise equal to the oracle's BF16 rounding of the exact FP64 sum
H_IDENTICAL_FRAC = 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


_cache = {}


def _setup(name, fp8=False):
    key = (name, fp8)
    if key not in _cache:
        from workload import make_inputs
        shape = A4_SHAPES[name]
        G.log(f"[setup a4{'+fp8' if fp8 else ''}] {name}: T={shape.T} E={shape.E} K={shape.K} I={shape.I} Lt={shape.Lt}")
        inp = make_inputs(shape)
        _cache[key] = (shape, inp, G.make_layer(shape, inp, T_max=shape.T, stage1_a4=True, stage2_fp8=fp8))
    return _cache[key]


def _z4(layer, shape, T):
    """GPU FP4 codes [T, Lt/2] and scales [T, Lt/32] of z, token order."""
    Lt = shape.Lt
    raw = layer.workspace_view(T, "z4", (T * Lt // 2 + T * Lt // 32,), torch.uint8).cpu().numpy()
    return raw[:T * Lt // 2].reshape(T, Lt // 2), raw[T * Lt // 2:].reshape(T, Lt // 32)


def _rest_from_h(shape, inp, run, h, fp8):
    """y, and out by the oracle from the given h (pair order) on."""
    ids = run.ids
    if fp8:
        hq, hs = O.fp8_quant(h)
        y = O.expert_down_fp8(hq, hs, ids, inp["down_codes"], inp["down_scales"])
    else:
        y = O.expert_down(h, ids, inp["down_codes"], inp["down_scales"])
    zc = O.combine(y, run.w.astype(np.float64))
    if shape.has_latent:
        ys = None
        if shape.S > 0:
            _, ys = O.shared(inp["x"], inp["sh_gate"], inp["sh_up"], inp["sh_down"])
        return y, O.output(zc, inp["w_up"], ys)
    return y, zc


def _check(name, fp8=False):
    shape, inp, layer = _setup(name, fp8)
    G.log(f"[a4 forward] {name}{' + fp8 second stage' if fp8 else ''}")
    return _check_run(shape, inp, layer, fp8)


def _check_run(shape, inp, layer, fp8):
    run = G.GpuRun(layer, shape, inp)
    G.check_routing_exact(run, shape.E, shape.K, run.logits)
    got = run.rows()
    ids = run.ids
    # FP4 codes and scales: bit-exact against the oracle's quantisation of the GPU's z
    zq, zs = _z4(layer, shape, shape.T)
    q_ref, s_ref = O.fp4_quant(got["z"])
    assert np.array_equal(zs, s_ref), f"{int(np.sum(zs != s_ref))} scale bytes differ"
    assert np.array_equal(zq, q_ref), f"{int(np.sum(zq != q_ref))} code bytes differ"
    nib = np.concatenate([zq & 0xF, zq >> 4])
    G.log(f"  z4: {zq.size * 2} codes, {zs.size} scales bit-exact "
          f"(saturated {int(np.sum((nib & 7) == 7))}, zero {int(np.sum((nib & 7) == 0))})")
    # h from those codes
    h_ref = O.expert_gateup_a4(zq, zs, ids, inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                               inp["up_scales"])
    G.assert_close("h (a4 stage)", G.bf16_f64(got["h"]), G.bf16_f64(h_ref))
    same = float(np.mean(got["h"] == h_ref))
    G.log(f"  h bitwise equal to the oracle: {same:.4%}")
    assert same >= H_IDENTICAL_FRAC
    # end to end from the GPU's h: every later step by the oracle
    y_ref, out_ref = _rest_from_h(shape, inp, run, got["h"], fp8)
    if not fp8:
        G.assert_close("y (from the GPU's h)", G.bf16_f64(got["y"]), G.bf16_f64(y_ref))
    G.assert_close_e2e("out (from the GPU's h, a4 stage)", G.bf16_f64(got["out"]), G.bf16_f64(out_ref))
    # fully independent: the oracle's own z decides its own codes. A code may then differ only in a
    # block whose BF16 z differs (an FP32 vs FP64 sum straddling a BF16 rounding midpoint), where the
    # E2M1 decision can land one step apart, so the output keeps the mean bar and at most
    # MAX_FLIP_FRAC of its elements may pass the max bar.
    ref = O.forward(inp, shape.K, ids_in=ids, want_intermediates=True, stage1_a4=True, stage2_fp8=fp8)
    nb = shape.Lt // 32
    zq_n = np.stack([zq & 0xF, zq >> 4], axis=2).reshape(shape.T, shape.Lt)
    rq_n = np.stack([ref["zq"] & 0xF, ref["zq"] >> 4], axis=2).reshape(shape.T, shape.Lt)
    code_blk = np.any((zq_n != rq_n).reshape(shape.T, nb, 32), axis=2) | (zs != ref["zs4"])
    z_blk = np.any((got["z"] != ref["z"]).reshape(shape.T, nb, 32), axis=2)
    G.log(f"  independent z: {int(z_blk.sum())}/{shape.T * nb} blocks with a BF16 difference, "
          f"{int(code_blk.sum())} with an FP4 code difference")
    assert not np.any(code_blk & ~z_blk), "FP4 codes differ in a block whose z is identical"
    og, orf = G.bf16_f64(got["out"]), G.bf16_f64(ref["out"])
    err = np.abs(og - orf)
    rms = float(np.sqrt(np.mean(orf * orf)))
    beyond = int(np.sum(err > G.MAX_REL_RMS * rms))
    G.log(f"  out (independent, a4 stage): max|err|={err.max():.3e} mean|err|={err.mean():.3e} "
          f"rms(ref)={rms:.3e} beyond-bar={beyond}/{err.size}")
    assert err.mean() <= G.MEAN_REL_RMS * rms
    assert beyond <= G.MAX_FLIP_FRAC * err.size
    return shape, inp, layer, run


@pytest.mark.parametrize("name", list(A4_SHAPES))
def test_a4_stage_parity(name):
    _check(name)


def test_a4_with_fp8_second_stage():
    _check("prefill_small", fp8=True)


@pytest.mark.parametrize("name,T", [("mid", 1), ("mid", 2), ("mid", 17), ("prefill_small", 128),
                                    ("prefill_small", 131), ("prefill_small", 257)])
def test_quantised_stages_ragged_token_counts(name, T):
    """Both quantised stages on a prefix of T tokens: 16-row expert tiles (mid) and, around the
    128-row tile threshold, ragged last tiles of 1-8 fragments (prefill_small)."""
    shape, inp, layer = _setup(name, fp8=True)
    sub = dict(inp, x=inp["x"][:T])
    G.log(f"[a4+fp8 ragged] {name} T={T}")
    _check_run(replace(shape, T=T), sub, layer, True)


@pytest.mark.parametrize("name", ["tiny", "prefill_small"])
def test_a4_stage_route_forward_bit_identical(name):
    shape, inp, layer = _setup(name)
    run = G.GpuRun(layer, shape, inp)
    G.check_fused_identical(layer, shape, inp, run)
