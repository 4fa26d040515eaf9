"""Pins for the oracle's number formats: E2M1, E8M0, MX dequantisation, BF16 rounding."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import _np_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_value_set():
    # The 16 E2M1 values are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; codes 0..7 positive in increasing
    # order, 8..15 their negatives (sign bit 3).
    pos = [O.e2m1(c) for c in range(8)]
    neg = [O.e2m1(c) for c in range(8, 16)]
    assert pos == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert neg == [-v for v in pos]
    assert math.copysign(1.0, O.e2m1(8)) == -1.0 and math.copysign(1.0, O.e2m1(0)) == 1.0
    assert sorted(set(abs(v) for v in pos + neg)) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_closed_form_all_codes():
    for e in range(255):
        assert O.e8m0(e) == math.ldexp(1.0, e - 127)
    assert math.isnan(O.e8m0(255))


def _golden_blocks():
    rows = []
    with open(os.path.join(GOLDEN, "mxfp4_blocks.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            sc, codes, vals = (p.strip() for p in line.split("|"))
            rows.append((int(sc), bytes.fromhex(codes), [float(v) for v in vals.split()]))
    return rows


def test_dequant_golden_blocks():
    blocks = _golden_blocks()
    assert len(blocks) == 4
    for sc, codes, vals in blocks:
        assert len(codes) == 16 and len(vals) == 32
        got = O.dequant(np.frombuffer(codes, np.uint8)[None, :], np.array([[sc]], np.uint8))[0]
        for g, v in zip(got, vals):
            assert g == v and math.copysign(1, g) == math.copysign(1, v), (sc, codes.hex(), got)


def test_dequant_golden_scale_axis():
    with open(os.path.join(GOLDEN, "mxfp4_scale_axis.txt")) as f:
        rows = [line.split("|") for line in f if not line.startswith("#") and line.strip()]
    codes = np.full((2, 32), 0x22, np.uint8)
    scales = np.array([[int(s) for s in r[1].split()] for r in rows], np.uint8)
    got = O.dequant(codes, scales)
    for i, r in enumerate(rows):
        assert np.all(got[i, :32] == float(r[2])) and np.all(got[i, 32:] == float(r[3]))


def test_dequant_matches_value_table_random():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, (7, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, (7, 4), dtype=np.uint8)
    a = O.dequant(codes, scales)
    b = R.dequant_table(codes, scales)
    assert np.array_equal(a, b) and np.array_equal(np.signbit(a), np.signbit(b))


def test_dequant_products_exact_in_bf16():
    # E2M1 has at most two significant bits, so with scales in [120, 124] every product is a
    # BF16 value: rounding to BF16 must leave it unchanged.
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256).repeat(5, 0)
    scales = np.repeat(np.arange(120, 125, dtype=np.uint8)[:, None], 16, 1)
    v = O.dequant(codes, scales)
    assert np.array_equal(O.bf16_to_f64(O.f64_to_bf16(v)), v)


def test_bf16_rne_halfway_and_double_rounding():
    f = O.lib().or_double_to_bf16
    assert f(1.0 + 2.0 ** -8) == 0x3F80            # exact tie -> even (1.0)
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82        # exact tie -> even (1 + 2^-6)
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81   # just above the tie: up (no double rounding)
    assert f(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    assert f(0.0) == 0x0000 and f(-0.0) == 0x8000
    assert f(2.0 ** -133) == 0x0001                # smallest subnormal
    assert f(3.0e38) == 0x7F62 and f(3.5e38) == 0x7F80   # largest finite region / overflow
    assert f(float("inf")) == 0x7F80 and f(float("nan")) & 0x7F80 == 0x7F80


def test_bf16_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    v32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(v32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rne_matches_bit_rounding_on_doubles():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))
    assert np.array_equal(O.f64_to_bf16(v), R.bf16_rne(v))


@pytest.mark.parametrize("bits", [0x0000, 0x3F80, 0xC0C0, 0x0001, 0x7F7F, 0x8000])
def test_bf16_to_double_exact(bits):
    ref = torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    assert O.lib().or_bf16_to_double(bits) == float(ref.to(torch.float64)[0])
