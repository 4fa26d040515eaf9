"""GPU parity at the full workload sizes: one GPU's TP8 share at decode (64 tokens) and prefill
(8192 tokens, Zipf-skewed), the full block (16384 tokens, Zipf, 1% exact rank-16/17 ties) and the
full unsharded experts (4096 tokens, intermediate 3072). Routing is compared bit for bit on every
token; floating-point tensors on a seeded token sample that the oracle computes one by one. The
fused route + forward call must reproduce the separate calls bit for bit at every size. A ragged
prefill (8000 tokens) runs the dense products with their last row tile shifted back over its
neighbour, in the output product's 256 x 224 tiling."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_helpers as G
from workload import SHAPES, make_inputs, sample_tokens, tie_tokens

pytestmark = pytest.mark.gpu

FULL = [("tp8_decode_t64", None), ("tp8_prefill_t8192", 48), ("tp8_block_t16384", 40),
        ("full_experts_t4096", 64)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()
    yield


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,n_sample", FULL)
def test_full_size_parity(name, n_sample):
    shape = SHAPES[name]
    G.log(f"[full] {name}: T={shape.T} H={shape.H} Lt={shape.Lt} E={shape.E} K={shape.K} I={shape.I}")
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=shape.T)
    run = G.GpuRun(layer, shape, inp)
    again = G.GpuRun(layer, shape, inp)
    assert torch.equal(again._out.view(torch.int16), run._out.view(torch.int16)), "second run differs"
    assert np.array_equal(again.ids, run.ids) and np.array_equal(again.inv, run.inv)
    del again
    G.log("  a second run: bit-identical")
    G.check_fused_identical(layer, shape, inp, run)
    G.log("  route_forward: bit-identical to route + forward")
    tokens = None if n_sample is None else sample_tokens(shape, n_sample)
    tied_logits = None
    if shape.tie_frac > 0:
        tt = tie_tokens(shape)
        lg = run.logits.copy()
        order = O.select(lg[tt].astype(np.float64), shape.K + 1)
        e16, e17 = order[:, shape.K - 1], order[:, shape.K]
        lg[tt, e17] = lg[tt, e16]
        run = G.GpuRun(layer, shape, inp, logits_in=lg)
        lo, hi = np.minimum(e16, e17), np.maximum(e16, e17)
        for i, t in enumerate(tt):
            assert lo[i] in run.ids[t] and hi[i] not in run.ids[t]
        G.log(f"  {len(tt)} tied tokens, {int(np.sum(e17 < e16))} change their selection")
        tied_logits = lg
        tokens = np.union1d(tokens, tt[:12])
    active = int(np.sum(run.counts > 0))
    G.log(f"  active experts {active}/{shape.E}, max load {int(run.counts.max())}")
    G.check_forward(shape, inp, run, oracle_logits_in=tied_logits, tokens=tokens)
    layer.close()
    del layer, run
    torch.cuda.empty_cache()


@pytest.mark.timeout(400)
def test_ragged_prefill_shifted_last_row_tile():
    """8000 tokens at the prefill shape: 32 row tiles of 256 with the last one starting at row 7744,
    so rows 7744..7935 are computed by two workgroups; the output product still takes 256 x 224 tiles
    (1024 tiles in four rounds against 896 of 256 x 256). The sample includes rows of the overlap,
    the last row and rows next to the tile boundaries."""
    shape = replace(SHAPES["tp8_prefill_t8192"], T=8000, name="tp8_prefill_t8000")
    G.log(f"[full] {shape.name}: T={shape.T}")
    inp = make_inputs(shape)
    layer = G.make_layer(shape, inp, T_max=shape.T)
    run = G.GpuRun(layer, shape, inp)
    G.check_fused_identical(layer, shape, inp, run)
    tokens = np.union1d(sample_tokens(shape, 24), [0, 255, 256, 7679, 7680, 7743, 7744, 7800, 7935, 7936, 7999])
    G.check_forward(shape, inp, run, tokens=tokens)
    layer.close()
    del layer, run
    torch.cuda.empty_cache()
