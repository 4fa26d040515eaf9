"""Python access to the FP64 CPU oracle in ``oracle.c`` (ctypes, numpy arrays).

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the bench's CPU-baseline
leg, never by the product path. It shares no code with the HIP library.

``forward`` composes the oracle's steps in the order the layer applies them (router, top-K,
gate weights, grouping by expert, latent down-projection, routed GLU experts, gate-weighted
combine, shared experts, up-projection plus shared add); each step is one C function whose
header cites the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (strict IEEE: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        sig = {
            "or_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "or_double_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "or_e2m1": (ctypes.c_double, [ctypes.c_int]),
            "or_e8m0": (ctypes.c_double, [ctypes.c_int]),
            "or_dequant": (None, [P, P, I64, I64, P]),
            "or_logits": (None, [P, I64, I64, P, I64, P, P]),
            "or_select": (None, [P, I64, I64, I64, P]),
            "or_route_weights": (None, [P, P, I64, I64, I64, P]),
            "or_permute": (None, [P, I64, I64, I64, P, P, P, P]),
            "or_latent_down": (None, [P, I64, I64, P, I64, P]),
            "or_shared": (None, [P, I64, I64, P, P, P, I64, I64, P, P]),
            "or_output": (None, [P, I64, I64, P, I64, P, P]),
            "or_experts": (None, [P, I64, I64, P, I64, I64, P, P, P, P, P, P, P, P]),
            "or_combine": (None, [P, P, I64, I64, I64, P]),
            "or_e4m3": (ctypes.c_double, [ctypes.c_int]),
            "or_fp8_quant": (None, [P, I64, I64, P, P]),
            "or_expert_down_fp8": (None, [P, P, I64, I64, I64, I64, P, P, P, P]),
            "or_fp4_quant": (None, [P, I64, I64, P, P]),
            "or_expert_gateup_a4": (None, [P, P, I64, I64, P, I64, I64, P, P, P, P, P]),
            "or_num_threads": (ctypes.c_int, []),
            "or_expert_down": (None, [P, I64, I64, I64, I64, P, P, P, P]),
            "or_shared_down": (None, [P, I64, I64, I64, P, I64, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ element formats

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = _c(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    f = np.vectorize(lambda s: lib().or_double_to_bf16(float(s)), otypes=[np.uint16])
    return f(v) if v.size else np.zeros(v.shape, np.uint16)


def num_threads() -> int:
    return int(lib().or_num_threads())


def e2m1(code: int) -> float:
    return lib().or_e2m1(int(code))


def e8m0(e: int) -> float:
    return lib().or_e8m0(int(e))


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (N, K // 32)
    out = np.empty((N, K), np.float64)
    lib().or_dequant(_p(codes), _p(scales), N, K, _p(out))
    return out


# ------------------------------------------------------------------ routing

def logits(x, w_router, bias=None) -> np.ndarray:
    x = _c(x, np.uint16)
    w = _c(w_router, np.uint16)
    T, Hin = x.shape
    E = w.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float64)
    lib().or_logits(_p(x), T, Hin, _p(w), E, _p(b), _p(out))
    return out


def select(lg: np.ndarray, K: int) -> np.ndarray:
    lg = _c(lg, np.float64)
    T, E = lg.shape
    ids = np.empty((T, K), np.int32)
    lib().or_select(_p(lg), T, E, K, _p(ids))
    return ids


def route_weights(lg: np.ndarray, ids: np.ndarray) -> np.ndarray:
    lg = _c(lg, np.float64)
    ids = _c(ids, np.int32)
    T, E = lg.shape
    K = ids.shape[1]
    w = np.empty((T, K), np.float64)
    lib().or_route_weights(_p(lg), _p(ids), T, E, K, _p(w))
    return w


@dataclass
class Permutation:
    counts: np.ndarray
    offsets: np.ndarray
    sorted_pairs: np.ndarray
    inv: np.ndarray


def permute(ids: np.ndarray, E: int) -> Permutation:
    ids = _c(ids, np.int32)
    T, K = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    lib().or_permute(_p(ids), T, K, E, _p(counts), _p(offsets), _p(sp), _p(inv))
    return Permutation(counts, offsets, sp, inv)


# ------------------------------------------------------------------ dense parts / experts

def latent_down(x, w_down) -> np.ndarray:
    x = _c(x, np.uint16)
    w = _c(w_down, np.uint16)
    T, H = x.shape
    Lt = w.shape[0]
    z = np.empty((T, Lt), np.uint16)
    lib().or_latent_down(_p(x), T, H, _p(w), Lt, _p(z))
    return z


def shared(x, sh_gate, sh_up, sh_down):
    x = _c(x, np.uint16)
    sg, su, sd = (_c(a, np.uint16) for a in (sh_gate, sh_up, sh_down))
    T, H = x.shape
    S, Is = sg.shape[0], sg.shape[1]
    hs = np.empty((T, S * Is), np.uint16)
    ys = np.empty((T, H), np.float64)
    lib().or_shared(_p(x), T, H, _p(sg), _p(su), _p(sd), S, Is, _p(hs), _p(ys))
    return hs, ys


def output(zc, w_up, ys=None) -> np.ndarray:
    zc = _c(zc, np.uint16)
    w = _c(w_up, np.uint16)
    T, Lt = zc.shape
    H = w.shape[0]
    ys = None if ys is None else _c(ys, np.float64)
    out = np.empty((T, H), np.uint16)
    lib().or_output(_p(zc), T, Lt, _p(w), H, _p(ys), _p(out))
    return out


def experts(z, ids, gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales,
            want_h: bool = True):
    z = _c(z, np.uint16)
    ids = _c(ids, np.int32)
    T, Lt = z.shape
    K = ids.shape[1]
    I = gate_codes.shape[1]
    arrs = [_c(a, np.uint8) for a in (gate_codes, gate_scales, up_codes, up_scales,
                                      down_codes, down_scales)]
    h = np.empty((T * K, I), np.uint16) if want_h else None
    y = np.empty((T * K, Lt), np.uint16)
    lib().or_experts(_p(z), T, Lt, _p(ids), K, I, *[_p(a) for a in arrs], _p(h), _p(y))
    return h, y


def expert_down(h, ids, down_codes, down_scales) -> np.ndarray:
    """y by pair id from given h (pair order) -- the down half of `experts`."""
    h = _c(h, np.uint16)
    ids = _c(ids, np.int32)
    T, K = ids.shape
    I = h.shape[1]
    Lt = down_codes.shape[1]
    dc, ds = _c(down_codes, np.uint8), _c(down_scales, np.uint8)
    y = np.empty((T * K, Lt), np.uint16)
    lib().or_expert_down(_p(h), T, K, I, Lt, _p(ids), _p(dc), _p(ds), _p(y))
    return y


def e4m3(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for S.1111.111)."""
    return lib().or_e4m3(int(code))


def fp8_quant(h) -> tuple[np.ndarray, np.ndarray]:
    """MX FP8 quantisation of BF16 rows [R, I]: (E4M3 codes [R, I], E8M0 scale bytes [R, I/32])."""
    h = _c(h, np.uint16)
    R, I = h.shape
    codes = np.empty((R, I), np.uint8)
    scales = np.empty((R, I // 32), np.uint8)
    lib().or_fp8_quant(_p(h), R, I, _p(codes), _p(scales))
    return codes, scales


def fp8_dequant(codes, scales) -> np.ndarray:
    """Values of MX FP8 rows: code value times its block's scale (FP64)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    table = np.array([e4m3(c) for c in range(256)], np.float64)
    return table[codes] * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def expert_down_fp8(hq, hs, ids, down_codes, down_scales) -> np.ndarray:
    """y by pair id from quantised h (pair order) -- the FP8 second stage."""
    hq = _c(hq, np.uint8)
    hs = _c(hs, np.uint8)
    ids = _c(ids, np.int32)
    T, K = ids.shape
    I = hq.shape[1]
    Lt = down_codes.shape[1]
    dc, ds = _c(down_codes, np.uint8), _c(down_scales, np.uint8)
    y = np.empty((T * K, Lt), np.uint16)
    lib().or_expert_down_fp8(_p(hq), _p(hs), T, K, I, Lt, _p(ids), _p(dc), _p(ds), _p(y))
    return y


def fp4_quant(z) -> tuple[np.ndarray, np.ndarray]:
    """MX FP4 quantisation of BF16 rows [R, L]: (E2M1 codes packed two per byte [R, L/2],
    E8M0 scale bytes [R, L/32]) -- the A4W4 first stage's activations (oracle.c, O11)."""
    z = _c(z, np.uint16)
    R, L = z.shape
    codes = np.empty((R, L // 2), np.uint8)
    scales = np.empty((R, L // 32), np.uint8)
    lib().or_fp4_quant(_p(z), R, L, _p(codes), _p(scales))
    return codes, scales


def expert_gateup_a4(zq, zs, ids, gate_codes, gate_scales, up_codes, up_scales) -> np.ndarray:
    """h by pair id from MX FP4 z (token order) -- the A4W4 first stage."""
    zq = _c(zq, np.uint8)
    zs = _c(zs, np.uint8)
    ids = _c(ids, np.int32)
    T, K = ids.shape
    Lt = zq.shape[1] * 2
    I = gate_codes.shape[1]
    arrs = [_c(a, np.uint8) for a in (gate_codes, gate_scales, up_codes, up_scales)]
    h = np.empty((T * K, I), np.uint16)
    lib().or_expert_gateup_a4(_p(zq), _p(zs), T, Lt, _p(ids), K, I, *[_p(a) for a in arrs], _p(h))
    return h


def shared_down(hs, sh_down) -> np.ndarray:
    """sum over shared experts of h_s . Wd_s^T (FP64) from given h_s -- the down half of `shared`."""
    hs = _c(hs, np.uint16)
    sd = _c(sh_down, np.uint16)
    T = hs.shape[0]
    S, H, Is = sd.shape
    ys = np.empty((T, H), np.float64)
    lib().or_shared_down(_p(hs), T, S, Is, _p(sd), H, _p(ys))
    return ys


def combine(y, w) -> np.ndarray:
    y = _c(y, np.uint16)
    w = _c(w, np.float64)
    T, K = w.shape
    Lt = y.shape[1]
    zc = np.empty((T, Lt), np.uint16)
    lib().or_combine(_p(y), _p(w), T, K, Lt, _p(zc))
    return zc


# ------------------------------------------------------------------ whole layer

def forward(inp: dict, K: int, logits_in=None, ids_in=None, want_intermediates=True,
            stage2_fp8: bool = False, stage1_a4: bool = False) -> dict:
    """Whole routed-expert forward on the tokens of ``inp["x"]``.

    ``logits_in`` replaces the router product (as the library's logits input does);
    ``ids_in`` forces the expert selection (the floating-point parity protocol uses the
    selection that was already checked bit-exactly, so a near-tie cannot mask a numeric
    comparison). ``stage2_fp8`` runs the down product on MX FP8 h (oracle.c, O10);
    ``stage1_a4`` runs the gate/up product on MX FP4 z (oracle.c, O11).
    Returns logits, ids, w, perm, z, zq / zs4 (FP4 codes and scales, or None), h, hq / hs8
    (FP8 codes and scales, or None), y (pair order), zc, hs, ys, out.
    """
    x = inp["x"]
    has_latent = "w_down" in inp
    lg = logits(x, inp["w_router"], inp.get("router_bias")) if logits_in is None \
        else _c(logits_in, np.float64)
    ids = select(lg, K) if ids_in is None else _c(ids_in, np.int32)
    w = route_weights(lg, ids)
    E = inp["w_router"].shape[0]
    perm = permute(ids, E)
    z = latent_down(x, inp["w_down"]) if has_latent else _c(x, np.uint16)
    h, y = experts(z, ids, inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                   inp["up_scales"], inp["down_codes"], inp["down_scales"],
                   want_h=want_intermediates or stage2_fp8)
    zq = zs4 = None
    if stage1_a4:    # first stage on MX FP4 z instead of BF16 z
        zq, zs4 = fp4_quant(z)
        h = expert_gateup_a4(zq, zs4, ids, inp["gate_codes"], inp["gate_scales"], inp["up_codes"],
                             inp["up_scales"])
        y = expert_down(h, ids, inp["down_codes"], inp["down_scales"])
    hq = hs8 = None
    if stage2_fp8:   # second stage on MX FP8 h instead of BF16 h
        hq, hs8 = fp8_quant(h)
        y = expert_down_fp8(hq, hs8, ids, inp["down_codes"], inp["down_scales"])
    zc = combine(y, w)
    hs = ys = None
    if has_latent:
        if "sh_gate" in inp and inp["sh_gate"].shape[0] > 0:
            hs, ys = shared(x, inp["sh_gate"], inp["sh_up"], inp["sh_down"])
        out = output(zc, inp["w_up"], ys)
    else:
        out = zc
    return dict(logits=lg, ids=ids, w=w, perm=perm, z=z, zq=zq, zs4=zs4, h=h, hq=hq, hs8=hs8, y=y, zc=zc,
                hs=hs, ys=ys, out=out)
