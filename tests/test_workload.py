"""Checks of the seeded input generator (workload/gen.py): the same seed gives the same bytes, each
tensor has its own stream, the values follow the stated distributions, the Zipf(1.1) routing bias is
the log of the Zipf pmf over a seeded permutation of the experts and skews the expert loads as the
skewed workloads require (uneven loads, experts with no tokens), and the tie and sample token sets
have the stated sizes."""
import math

import numpy as np
import torch

from workload import SHAPES, make_inputs, sample_tokens, tie_tokens
from workload.gen import ZIPF_S, LayerShape, zipf_bias, _rngs

MID = LayerShape("mid", 200, 1024, 512, 64, 8, 256, 2, 128, True, "zipf", 0.0, 7)


def _f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_same_seed_same_bytes_and_independent_streams():
    a, b = make_inputs(MID), make_inputs(MID)
    assert a.keys() == b.keys()
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert np.array_equal(a[k], b[k]), k
    # asking for a subset draws the same values (each tensor has a stream of its own)
    sub = make_inputs(MID, ["down_codes", "x"])
    assert np.array_equal(sub["x"], a["x"]) and np.array_equal(sub["down_codes"], a["down_codes"])
    # another seed gives other values
    other = make_inputs(LayerShape(**{**MID.__dict__, "seed": 8}))
    assert not np.array_equal(other["x"], a["x"])


def test_distributions_follow_the_configs():
    inp = make_inputs(MID)
    x = _f64(inp["x"])
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    for name, fan_in in (("w_router", MID.Hin), ("w_down", MID.H), ("w_up", MID.Lt), ("sh_gate", MID.H),
                         ("sh_down", MID.Is)):
        w = _f64(inp[name])
        assert abs(w.std() * math.sqrt(fan_in) - 1.0) < 0.03, name
    codes = np.concatenate([inp[k].ravel() for k in ("gate_codes", "up_codes", "down_codes")])
    hist = np.bincount(codes, minlength=256)
    assert hist.min() > 0.8 * codes.size / 256 and hist.max() < 1.2 * codes.size / 256
    for nib in (codes & 0xF, codes >> 4):   # both nibbles uniform over all 16 E2M1 codes
        h = np.bincount(nib, minlength=16)
        assert h.min() > 0.95 * nib.size / 16 and h.max() < 1.05 * nib.size / 16
    scales = np.concatenate([inp[k].ravel() for k in ("gate_scales", "up_scales", "down_scales")])
    assert scales.min() == 120 and scales.max() == 124
    h = np.bincount(scales - 120, minlength=5)
    assert h.min() > 0.95 * scales.size / 5 and h.max() < 1.05 * scales.size / 5


def test_zipf_bias_is_log_pmf_over_a_seeded_permutation():
    E = 896
    b = zipf_bias(E, _rngs(2)["zipf_rank"]).astype(np.float64)
    pmf = np.arange(1, E + 1, dtype=np.float64) ** (-ZIPF_S)
    pmf /= pmf.sum()
    assert np.allclose(np.sort(np.exp(b))[::-1], pmf, rtol=1e-6)
    assert abs(np.exp(b).sum() - 1.0) < 1e-5
    assert np.array_equal(b, zipf_bias(E, _rngs(2)["zipf_rank"]).astype(np.float64))
    assert SHAPES["tp8_prefill_t8192"].routing == "zipf" and SHAPES["tp8_decode_t64"].routing == "uniform"


def test_zipf_skew_gives_uneven_loads_and_empty_experts():
    """Routing simulated at the prefill workload's shape: logits of unit spread (x ~ N(0,1) times a
    router of variance 1/fan_in) plus the bias, top-16 of 896 for 8192 tokens."""
    s = SHAPES["tp8_prefill_t8192"]
    bias = zipf_bias(s.E, _rngs(s.seed)["zipf_rank"]).astype(np.float64)
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((s.T, s.E)) + bias
    top = np.argpartition(-logits, s.K, axis=1)[:, :s.K]
    load = np.bincount(top.ravel(), minlength=s.E)
    active = int(np.sum(load > 0))
    assert 300 < active < 460, active                   # uneven: well under 896 experts see tokens
    assert load.max() > 20 * load[load > 0].mean()      # a few experts take most pairs
    # uniform routing, for contrast: every expert is used at this many tokens
    top_u = np.argpartition(-rng.standard_normal((s.T, s.E)), s.K, axis=1)[:, :s.K]
    assert np.all(np.bincount(top_u.ravel(), minlength=s.E) > 0)


def test_tie_and_sample_token_sets():
    blk = SHAPES["tp8_block_t16384"]
    tt = tie_tokens(blk)
    assert len(tt) == math.ceil(0.01 * blk.T) == 164
    assert np.all(np.diff(tt) > 0) and tt[0] >= 0 and tt[-1] < blk.T
    assert np.array_equal(tt, tie_tokens(blk))
    assert len(tie_tokens(SHAPES["tp8_prefill_t8192"])) == 0
    sm = sample_tokens(SHAPES["tp8_prefill_t8192"], 256)
    assert len(sm) == 256 and np.all(np.diff(sm) > 0) and sm[-1] < 8192
    assert np.array_equal(sample_tokens(SHAPES["tp8_decode_t64"], 256), np.arange(64))
