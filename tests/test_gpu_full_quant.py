"""GPU parity of the quantised expert stages at the full sizes, in the launch configuration the
benchmark times: the TP8 share at 64-token decode (16-row expert tiles), 8192-token Zipf prefill
(128-row tiles) and the 16384-token block, with the A4W4 first stage (MX FP4 z) and the FP8 second
stage (MX FP8 h) together, and the A4W4 stage alone at prefill and on the full unsharded experts
(4096 tokens, intermediate 3072). Routing is compared bit for bit on every token; the quantised codes
and the floating-point stages on a seeded token sample that the oracle computes one by one:
- FP4 codes and scales of z, bit-exact against the oracle's quantisation of the GPU's z;
- h against the oracle's gate/up product on those codes;
- FP8 codes and scales of h, bit-exact against the oracle's quantisation of the GPU's h;
- y against the oracle's down product on those codes (or on the GPU's BF16 h);
- the output end to end from the GPU's h, and against the oracle's fully independent forward
  (mean bar; code differences only where the BF16 z or h already differs).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_helpers as G
from workload import SHAPES, make_inputs, sample_tokens

pytestmark = pytest.mark.gpu

# (workload, sampled tokens or all, FP8 second stage too). The FP8 stage keeps a 128-row tile of h in
# LDS and so needs I <= 512: the full unsharded experts (I = 3072) run the A4W4 stage alone.
CASES = [("tp8_decode_t64", None, True), ("tp8_prefill_t8192", 32, True), ("tp8_prefill_t8192", 32, False),
         ("tp8_block_t16384", 24, True), ("full_experts_t4096", 64, False)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


def _nibbles(codes: np.ndarray) -> np.ndarray:
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,n_sample,fp8", CASES)
def test_full_size_quantised_stages(name, n_sample, fp8):
    shape = SHAPES[name]
    T, K, Lt, I = shape.T, shape.K, shape.Lt, shape.I
    G.log(f"[full quant] {name}: A4W4 first stage{' + FP8 second stage' if fp8 else ''}")
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=T, stage1_a4=True, stage2_fp8=fp8)
    run = G.GpuRun(layer, shape, inp)
    again = G.GpuRun(layer, shape, inp)
    assert torch.equal(again._out.view(torch.int16), run._out.view(torch.int16)), "second run differs"
    del again
    G.check_routing_exact(run, shape.E, K, run.logits)
    tok = np.arange(T) if n_sample is None else sample_tokens(shape, n_sample)
    got = run.rows(tok)
    ids = run.ids[tok]
    G.log(f"  active experts {int(np.sum(run.counts > 0))}/{shape.E}, {len(tok)} tokens compared")

    raw = layer.workspace_view(T, "z4", (T * Lt // 2 + T * Lt // 32,), torch.uint8).cpu().numpy()
    zq = raw[:T * Lt // 2].reshape(T, Lt // 2)[tok]
    zs = raw[T * Lt // 2:].reshape(T, Lt // 32)[tok]
    q_ref, s_ref = O.fp4_quant(got["z"])
    assert np.array_equal(zs, s_ref) and np.array_equal(zq, q_ref), "FP4 z differs from the oracle's"
    h_ref = O.expert_gateup_a4(zq, zs, ids, inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                               inp["up_scales"])
    G.assert_close("h (a4 stage)", G.bf16_f64(got["h"]), G.bf16_f64(h_ref))

    P = T * K
    pairs = (tok[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    if fp8:
        raw8 = layer.workspace_view(T, "h8", (P * I + P * (I // 32),), torch.uint8).cpu().numpy()
        rows = run.inv[pairs]
        hq = raw8[:P * I].reshape(P, I)[rows]
        hs = raw8[P * I:].reshape(P, I // 32)[rows]
        q8, s8 = O.fp8_quant(got["h"])
        assert np.array_equal(hs, s8) and np.array_equal(hq, q8), "FP8 h differs from the oracle's"
        y_ref = O.expert_down_fp8(hq, hs, ids, inp["down_codes"], inp["down_scales"])
    else:
        y_ref = O.expert_down(got["h"], ids, inp["down_codes"], inp["down_scales"])
    G.assert_close("y", G.bf16_f64(got["y"]), G.bf16_f64(y_ref))

    sub = dict(inp, x=inp["x"][tok])
    zc_ref = O.combine(y_ref, run.w[tok].astype(np.float64))
    if shape.has_latent:
        ys = None
        if shape.S > 0:
            _, ys = O.shared(sub["x"], inp["sh_gate"], inp["sh_up"], inp["sh_down"])
        out_ref = O.output(zc_ref, inp["w_up"], ys)
    else:
        out_ref = zc_ref
    G.assert_close_e2e("out (from the GPU's h)", G.bf16_f64(got["out"]), G.bf16_f64(out_ref))

    ref = O.forward(sub, K, ids_in=ids, want_intermediates=True, stage1_a4=True, stage2_fp8=fp8)
    nb = Lt // 32
    code_blk = np.any((_nibbles(zq) != _nibbles(ref["zq"])).reshape(len(tok), nb, 32), axis=2) | (zs != ref["zs4"])
    z_blk = np.any((got["z"] != ref["z"]).reshape(len(tok), nb, 32), axis=2)
    G.log(f"  independent z: {int(z_blk.sum())} blocks with a BF16 difference, {int(code_blk.sum())} with a code difference")
    assert not np.any(code_blk & ~z_blk), "FP4 codes differ in a block whose z is identical"
    og, orf = G.bf16_f64(got["out"]), G.bf16_f64(ref["out"])
    err = np.abs(og - orf)
    rms = float(np.sqrt(np.mean(orf * orf)))
    beyond = int(np.sum(err > G.MAX_REL_RMS * rms))
    G.log(f"  out (independent): max|err|={err.max():.3e} mean|err|={err.mean():.3e} rms(ref)={rms:.3e} "
          f"beyond-bar={beyond}/{err.size}")
    assert err.mean() <= G.MEAN_REL_RMS * rms
    assert beyond <= G.MAX_FLIP_FRAC * err.size
    layer.close()
    del layer, run
    torch.cuda.empty_cache()
