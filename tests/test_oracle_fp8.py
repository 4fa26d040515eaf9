"""Pins of the oracle's FP8 second stage (oracle.c, O10): the E4M3 code table, the MX FP8
quantiser of h (reading F1: OCP MX FP8, one E8M0 scale per 32 values along I, shared exponent
floor(log2 amax) - 8, round to nearest even, saturation at 448) and the down product on the
quantised h (F2).

The pins do not re-derive the oracle's own arithmetic: the code table is checked against torch's
float8_e4m3fn (an independent library routine) and the OCP anchor values; the element rounding
against a brute-force nearest search over all finite codes and against torch's conversion; the
scale choice against its defining property (the block maximum lands in [256, 512) after
scaling); the down product against the BF16-stage oracle on inputs the FP8 format holds exactly.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as o

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16(x: np.ndarray) -> np.ndarray:
    return o.f64_to_bf16(np.asarray(x, np.float64))


def _torch_e4m3_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_table_matches_torch_float8():
    ours = np.array([o.e4m3(c) for c in range(256)])
    ref = _torch_e4m3_values()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_e4m3_anchor_values():
    # OCP MX v1.0, E4M3: largest normal 448, smallest normal 2^-6, smallest subnormal 2^-9,
    # NaN at S.1111.111, no infinities
    assert o.e4m3(0x7E) == 448.0 and o.e4m3(0xFE) == -448.0
    assert o.e4m3(0x08) == 2.0 ** -6 and o.e4m3(0x01) == 2.0 ** -9
    assert o.e4m3(0x38) == 1.0 and o.e4m3(0x40) == 2.0
    assert np.isnan(o.e4m3(0x7F)) and np.isnan(o.e4m3(0xFF))
    assert o.e4m3(0x80) == 0.0 and np.signbit(o.e4m3(0x80))
    finite = sorted({o.e4m3(c) for c in range(256) if not np.isnan(o.e4m3(c))})
    assert len(finite) == 253            # 254 finite codes, +0 and -0 equal


def _random_h(rng, R, I, spread=6.0):
    # per-block magnitudes spread over 2^+-spread, with zeros, sign mix and tiny elements
    mag = np.exp2(rng.uniform(-spread, spread, (R, I // 32, 1))) * rng.standard_normal((R, I // 32, 32))
    mag = mag.reshape(R, I)
    mag[rng.random((R, I)) < 0.03] = 0.0
    mag[rng.random((R, I)) < 0.03] *= 2.0 ** -12   # elements far below the block max (subnormal codes)
    return _bf16(mag)


def test_scale_puts_block_max_in_256_512():
    rng = np.random.default_rng(1)
    h = _random_h(rng, 24, 256)
    codes, scales = o.fp8_quant(h)
    hv = o.bf16_to_f64(h).reshape(24, 8, 32)
    amax = np.abs(hv).max(axis=2)
    X = scales.astype(np.int64) - 127
    scaled = amax / np.ldexp(1.0, X)
    nz = amax > 0
    assert np.all((scaled[nz] >= 256) & (scaled[nz] < 512))
    assert np.all(scales[~nz] == 0)


def test_elements_round_to_nearest_even_code_brute_force():
    rng = np.random.default_rng(2)
    h = _random_h(rng, 6, 64)
    codes, scales = o.fp8_quant(h)
    hv = o.bf16_to_f64(h)
    table = _torch_e4m3_values()
    pos = [c for c in range(0x7F)]                    # non-negative finite codes 0x00..0x7E
    for r in range(hv.shape[0]):
        for i in range(hv.shape[1]):
            X = int(scales[r, i // 32]) - 127
            a = abs(hv[r, i]) / 2.0 ** X
            d = [abs(table[c] - a) for c in pos]
            best = min(d)
            cands = [c for c in pos if d[pos.index(c)] == best]
            if a > 448:                                # saturation
                want = 0x7E
            elif len(cands) == 1:
                want = cands[0]
            else:                                      # tie: even mantissa
                want = [c for c in cands if c % 2 == 0][0]
            sign = 0x80 if np.signbit(hv[r, i]) else 0
            assert codes[r, i] == (want | sign), (r, i, hv[r, i], X, codes[r, i], want)


def test_elements_match_torch_conversion():
    rng = np.random.default_rng(3)
    h = _random_h(rng, 64, 512, spread=20.0)
    codes, scales = o.fp8_quant(h)
    hv = o.bf16_to_f64(h)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    q = np.clip(hv / np.ldexp(1.0, X), -448.0, 448.0)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_saturation_zero_block_and_signed_zero():
    h = np.zeros((1, 64), np.float64)
    h[0, 0] = 1.9921875            # 2^0 (1 + 127/128): scaled max 510 -> saturates at 448
    h[0, 1] = -1.0
    h[0, 33] = -0.0                # second block: zeros only, one negative zero
    codes, scales = o.fp8_quant(_bf16(h))
    assert scales[0, 0] == 127 - 8 and codes[0, 0] == 0x7E
    assert codes[0, 1] == (0x80 | 0x78)            # -1 * 2^8 = -256: exponent field 15, mantissa 0
    assert scales[0, 1] == 0 and np.all(codes[0, 32:] == np.where(np.arange(32) == 1, 0x80, 0))


def test_fp8_representable_h_round_trips_exactly():
    rng = np.random.default_rng(4)
    table = _torch_e4m3_values()
    R, I = 8, 128
    cq = rng.integers(0, 0x7F, (R, I)).astype(np.uint8) | (rng.integers(0, 2, (R, I)) << 7).astype(np.uint8)
    for r in range(R):
        for b in range(I // 32):
            cq[r, b * 32 + rng.integers(0, 32)] = 0x78 + rng.integers(0, 7)   # block max in [256, 448]
    s = rng.integers(110, 140, (R, I // 32)).astype(np.uint8)
    h = table[cq] * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    hb = _bf16(h)
    assert np.array_equal(o.bf16_to_f64(hb), h)    # E4M3 values scaled by 2^X are BF16 values
    codes, scales = o.fp8_quant(hb)
    assert np.array_equal(scales, s)
    assert np.array_equal(o.fp8_dequant(codes, scales), h)


def test_quantisation_error_bound():
    rng = np.random.default_rng(5)
    h = _random_h(rng, 32, 256)
    codes, scales = o.fp8_quant(h)
    hv = o.bf16_to_f64(h)
    dq = o.fp8_dequant(codes, scales)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    scaled = np.abs(hv) / np.ldexp(1.0, X)
    ok = scaled <= 448
    # half a unit in the last of 4 significant bits, or half the subnormal quantum 2^-9
    bound = np.maximum(np.abs(hv) * 2.0 ** -4, np.ldexp(1.0, X - 10))
    assert np.all(np.abs(dq - hv)[ok] <= bound[ok])
    assert np.all(np.abs(dq[~ok]) == 448 * np.ldexp(1.0, X[~ok]))


def test_fp8_down_equals_bf16_down_when_h_is_representable():
    rng = np.random.default_rng(6)
    T, K, E, I, Lt = 3, 2, 4, 64, 32
    table = _torch_e4m3_values()
    cq = rng.integers(0, 0x7F, (T * K, I)).astype(np.uint8) | (rng.integers(0, 2, (T * K, I)) << 7).astype(np.uint8)
    cq[:, 0] = 0x78
    cq[:, 32] = 0x7D
    s = rng.integers(115, 125, (T * K, I // 32)).astype(np.uint8)
    h = _bf16(table[cq] * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1))
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    dc = rng.integers(0, 256, (E, Lt, I // 2)).astype(np.uint8)
    ds = rng.integers(120, 130, (E, Lt, I // 32)).astype(np.uint8)
    y_bf16 = o.expert_down(h, ids, dc, ds)
    hq, hs = o.fp8_quant(h)
    y_fp8 = o.expert_down_fp8(hq, hs, ids, dc, ds)
    assert np.array_equal(y_bf16, y_fp8)
    # and a changed code changes the result (the quantised input is really read)
    hq2 = hq.copy()
    hq2[0, 5] ^= 0x08
    assert not np.array_equal(o.expert_down_fp8(hq2, hs, ids, dc, ds)[0], y_fp8[0])
