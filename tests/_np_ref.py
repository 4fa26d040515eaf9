"""Independent numpy formulations used to pin the oracle (tests only).

Each helper reaches the same quantity as an oracle function by a different route: a value table
instead of a bit decode, float64 bit manipulation instead of frexp/nearbyint, library matmuls
instead of index loops, a dense all-experts-masked sum instead of a per-pair gather.
"""
import numpy as np
import scipy.special

# E2M1 value set +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, listed in code order 0..15 (OCP bit map).
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_rne(v):
    """float64 -> BF16 bits by integer RNE on the float64 bit pattern (normal range only)."""
    v = np.ascontiguousarray(v, np.float64)
    b = v.view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint32)
    ex = ((b >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    mant = b & np.uint64((1 << 52) - 1)
    keep = (mant >> np.uint64(45)).astype(np.int64)
    rem = (mant & np.uint64((1 << 45) - 1)).astype(np.uint64)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & 1) == 1))
    keep = keep + up.astype(np.int64)
    ex = ex + (keep >> 7)
    keep = keep & 0x7F
    ebf = ex - 1023 + 127
    zero = (v == 0)
    assert np.all(zero | ((ebf >= 1) & (ebf <= 254))), "outside the BF16 normal range"
    bits = (sign << 15) | (np.where(zero, 0, ebf).astype(np.uint32) << 7) | \
        np.where(zero, 0, keep).astype(np.uint32)
    return bits.astype(np.uint16)


def dequant_table(codes, scales):
    """MX matrix [N, K] from codes [N, K/2] and scales [N, K/32] via the value table."""
    codes = np.asarray(codes, np.uint8)
    N, half = codes.shape
    vals = np.empty((N, 2 * half))
    vals[:, 0::2] = E2M1_TABLE[codes & 0xF]
    vals[:, 1::2] = E2M1_TABLE[codes >> 4]
    sc = np.repeat(np.exp2(np.asarray(scales, np.float64) - 127.0), 32, axis=1)
    return vals * sc


def glu_mlp(z64, wg, wu, wd):
    """bf16(bf16(silu(z.wg^T) * (z.wu^T)) . wd^T) with float64 matmuls (row vectors z)."""
    g = z64 @ wg.T
    u = z64 @ wu.T
    h = bf16_rne(g * scipy.special.expit(g) * u)
    return h, bf16_rne(bf16_bits_to_f64(h) @ wd.T)


def topk_lexsort(lg, K):
    """Reference selection: stable full sort by (logit descending, index ascending)."""
    T, E = lg.shape
    idx = np.arange(E)
    return np.stack([np.lexsort((idx, -lg[t]))[:K] for t in range(T)]).astype(np.int32)


def masked_moe(z_bits, inp, lg, K):
    """Dense all-experts-masked formulation: zc_t = bf16(sum over slots of w * FFN_e(z_t)),
    evaluating every expert on every token and masking by the selection."""
    z64 = bf16_bits_to_f64(z_bits)
    T = z64.shape[0]
    E = inp["gate_codes"].shape[0]
    ids = topk_lexsort(lg, K)
    s = scipy.special.expit(lg)
    ffn = []
    for e in range(E):
        wg = dequant_table(inp["gate_codes"][e], inp["gate_scales"][e])
        wu = dequant_table(inp["up_codes"][e], inp["up_scales"][e])
        wd = dequant_table(inp["down_codes"][e], inp["down_scales"][e])
        ffn.append(bf16_bits_to_f64(glu_mlp(z64, wg, wu, wd)[1]))     # [T, Lt] for every token
    zc = np.empty((T, z64.shape[1]))
    for t in range(T):
        mask = np.zeros(E, bool)
        mask[ids[t]] = True
        denom = np.sum(s[t, ids[t]])
        acc = np.zeros(z64.shape[1])
        for e_ in ids[t]:                                 # slot order
            acc = acc + (s[t, e_] / denom) * ffn[e_][t] * mask[e_]
        zc[t] = acc
    return ids, bf16_rne(zc)
