"""Pins of the oracle's A4W4 first stage (oracle.c, O11): the MX FP4 quantiser of z (reading A1:
OCP MX FP4, one E8M0 scale per 32 values along the latent axis, shared exponent
floor(log2 amax) - 2, round to nearest even on the E2M1 grid, saturation at 6, sign kept, two codes
per byte with the even element in the low nibble) and the gate/up product on the quantised z (A2).

The pins do not re-derive the oracle's own arithmetic: the element rounding is checked against a
brute-force nearest search over the eight E2M1 magnitudes written out here, with ties sent to the
even code; the scale choice against its defining property (every non-zero block maximum lands in
[4, 8) after scaling); the packing against hand-derived bytes; the product against the BF16-stage
oracle on inputs the FP4 format holds exactly.
"""
import numpy as np
import pytest

from oracle import oracle as o

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# The E2M1 magnitudes of codes 0..7 (sign in bit 3), written out independently of the oracle.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _bf16(x: np.ndarray) -> np.ndarray:
    return o.f64_to_bf16(np.asarray(x, np.float64))


def _unpack(codes: np.ndarray) -> np.ndarray:
    """[R, L/2] packed bytes -> [R, L] 4-bit codes (element 2i = low nibble of byte i)."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def _values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = _unpack(codes)
    mag = E2M1[c & 7] * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    return np.where(c & 8, -mag, mag)


def _brute_code(a: float) -> int:
    """Nearest E2M1 magnitude code of a >= 0 (values past 6 saturate); ties to the even code."""
    d = np.abs(E2M1 - a)
    best = np.flatnonzero(d == d.min())
    return int(best[0] if len(best) == 1 else best[best % 2 == 0][0])


def test_scale_puts_block_max_in_4_8():
    rng = np.random.default_rng(1)
    z = _bf16(rng.standard_normal((6, 256)) * np.ldexp(1.0, rng.integers(-20, 20, (6, 1))))
    codes, scales = o.fp4_quant(z)
    zv = o.bf16_to_f64(z).reshape(6, 8, 32)
    amax = np.abs(zv).max(axis=2)
    X = scales.astype(np.int64) - 127
    scaled = amax / np.ldexp(1.0, X)
    assert np.all((scaled >= 4) & (scaled < 8))


def test_elements_round_to_nearest_even_code_brute_force():
    rng = np.random.default_rng(2)
    z = _bf16(rng.standard_normal((8, 128)) * 3.0)
    # plant exact ties of the E2M1 grid (in units of the block scale 2^X, X = 0 with a block max of 6)
    z[0, :32] = _bf16(np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -2.5, -5.0]
                               + [0.0] * 20))
    codes, scales = o.fp4_quant(z)
    c = _unpack(codes)
    zv = o.bf16_to_f64(z)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    for r in range(z.shape[0]):
        for k in range(z.shape[1]):
            a = abs(zv[r, k]) / 2.0 ** X[r, k]
            assert c[r, k] & 7 == _brute_code(a), (r, k, zv[r, k], X[r, k])
            assert (c[r, k] >> 3) == (z[r, k] >> 15)
    # the planted row: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4, 7 -> 6
    assert scales[0, 0] == 127
    assert list(c[0, :12]) == [7, 0, 2, 2, 4, 4, 6, 6, 7, 8, 12, 14]


def test_nibble_order_sign_and_zero_block():
    z = np.zeros((2, 64), np.uint16)
    z[0, 0] = _bf16(np.array([6.0]))[0]          # code 7 in the low nibble of byte 0
    z[0, 1] = _bf16(np.array([-1.0]))[0]         # code 8|2 in the high nibble
    z[0, 3] = 0x8000                              # -0 keeps its sign
    z[1, 32:] = 0x8000                            # an all-(-0) block
    codes, scales = o.fp4_quant(z)
    assert codes[0, 0] == 0xA7
    assert codes[0, 1] == 0x80
    assert scales[0, 0] == 127 and scales[0, 1] == 0      # X = 0; all-zero block X = -127
    assert scales[1, 0] == 0 and scales[1, 1] == 0
    assert np.all(codes[1, :16] == 0) and np.all(codes[1, 16:] == 0x88)


def test_fp4_representable_z_round_trips_exactly():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (5, 96))
    c[:, ::32] = 7                                # every block holds a 6: the scale is the one drawn
    X = rng.integers(-10, 10, (5, 3))
    vals = np.where(c & 8, -1.0, 1.0) * E2M1[c & 7] * np.repeat(np.ldexp(1.0, X), 32, axis=1)
    z = _bf16(vals)
    codes, scales = o.fp4_quant(z)
    assert np.array_equal(scales.astype(np.int64) - 127, X)
    assert np.array_equal(_values(codes, scales), o.bf16_to_f64(z))


def test_quantisation_error_bound():
    rng = np.random.default_rng(4)
    z = _bf16(rng.standard_normal((16, 128)) * np.ldexp(1.0, rng.integers(-6, 6, (16, 1))))
    codes, scales = o.fp4_quant(z)
    zv = o.bf16_to_f64(z)
    dq = _values(codes, scales)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    a = np.abs(zv) / np.ldexp(1.0, X)
    ok = a <= 6
    # half a unit in the last of 2 significant bits, or half the subnormal quantum 1/2
    lead = np.floor(np.log2(np.maximum(a, 1e-300)))
    quantum = np.ldexp(1.0, (np.maximum(lead - 1, -1) + X).astype(np.int64))
    assert np.all(np.abs(dq - zv)[ok] <= quantum[ok] / 2)
    assert np.all(np.abs(dq[~ok]) == 6 * np.ldexp(1.0, X[~ok]))


def test_a4_gateup_equals_bf16_gateup_when_z_is_representable():
    rng = np.random.default_rng(5)
    T, K, E, I, Lt = 3, 2, 4, 32, 64
    c = rng.integers(0, 16, (T, Lt))
    c[:, ::32] = 7
    z = _bf16(np.where(c & 8, -1.0, 1.0) * E2M1[c & 7]
              * np.repeat(np.ldexp(1.0, rng.integers(-3, 3, (T, Lt // 32))), 32, axis=1))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    gc = rng.integers(0, 256, (E, I, Lt // 2)).astype(np.uint8)
    gs = rng.integers(120, 128, (E, I, Lt // 32)).astype(np.uint8)
    uc = rng.integers(0, 256, (E, I, Lt // 2)).astype(np.uint8)
    us = rng.integers(120, 128, (E, I, Lt // 32)).astype(np.uint8)
    dc = rng.integers(0, 256, (E, Lt, I // 2)).astype(np.uint8)
    ds = rng.integers(120, 128, (E, Lt, I // 32)).astype(np.uint8)
    h_bf16, _ = o.experts(z, ids, gc, gs, uc, us, dc, ds)
    zq, zs = o.fp4_quant(z)
    h_a4 = o.expert_gateup_a4(zq, zs, ids, gc, gs, uc, us)
    assert np.array_equal(h_bf16, h_a4)
    # the quantised input is what is read: flipping one code's sign changes that token's h
    zq2 = zq.copy()
    zq2[1, 0] ^= 0x08
    h2 = o.expert_gateup_a4(zq2, zs, ids, gc, gs, uc, us)
    assert not np.array_equal(h2[K:2 * K], h_a4[K:2 * K]) and np.array_equal(h2[:K], h_a4[:K])


def test_forward_stage1_a4_composes_the_quantised_first_stage():
    rng = np.random.default_rng(6)
    T, K, E, I, Lt = 4, 2, 4, 32, 64
    inp = dict(
        x=_bf16(rng.standard_normal((T, Lt))),
        w_router=_bf16(rng.standard_normal((E, Lt)) / 8),
        gate_codes=rng.integers(0, 256, (E, I, Lt // 2)).astype(np.uint8),
        gate_scales=rng.integers(120, 125, (E, I, Lt // 32)).astype(np.uint8),
        up_codes=rng.integers(0, 256, (E, I, Lt // 2)).astype(np.uint8),
        up_scales=rng.integers(120, 125, (E, I, Lt // 32)).astype(np.uint8),
        down_codes=rng.integers(0, 256, (E, Lt, I // 2)).astype(np.uint8),
        down_scales=rng.integers(120, 125, (E, Lt, I // 32)).astype(np.uint8),
    )
    f = o.forward(inp, K, stage1_a4=True)
    zq, zs = o.fp4_quant(f["z"])
    assert np.array_equal(f["zq"], zq) and np.array_equal(f["zs4"], zs)
    h = o.expert_gateup_a4(zq, zs, f["ids"], inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                           inp["up_scales"])
    assert np.array_equal(f["h"], h)
    assert np.array_equal(f["y"], o.expert_down(h, f["ids"], inp["down_codes"], inp["down_scales"]))
    # random z is not FP4-representable: the A4W4 layer differs from the BF16 layer
    assert not np.array_equal(f["out"], o.forward(inp, K)["out"])
