"""The quantized GEMM oracle (oracle/quant_gemm.py) pinned to what the definitions fix: a
hand-worked example, integer arithmetic on exactly representable values, a brute-force loop on
tiny inputs, closed forms, and planted mistakes that must fail a pin.  CPU only."""
from __future__ import annotations

import itertools
import os

import numpy as np
import pytest

from oracle import quant_gemm as qg
from oracle.formats import decode_fp8_e4m3fn, fp8_e4m3fn_table

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_gemm_worked_example.txt")


def golden():
    out = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (p.strip() for p in line.split("=", 1))
                out[k] = [int(x, 16) if x.startswith("0x") else float(x) for x in v.split()]
    return out


def bf16_bits(x):
    """Exactly representable floats -> bf16 bits (the values used here need no rounding)."""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert ((u & 0xFFFF) == 0).all()
    return (u >> 16).astype(np.uint16)


def fp8_codes_of(values):
    """Codes of exactly representable e4m3fn values (looked up in the closed-form table)."""
    tab = fp8_e4m3fn_table()
    out = np.empty(np.shape(values), np.uint8)
    for idx, v in np.ndenumerate(np.asarray(values, np.float64)):
        c = [i for i in range(256) if tab[i] == v and not (v == 0 and i == 0x80)]
        assert c, v
        out[idx] = c[0]
    return out


def pack_int4(q):
    """int [N, K] in -8..7 -> bytes, low nibble = even k (the reading, restated for the test)."""
    q = np.asarray(q, np.int64) & 0xF
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- pins
def pin_worked_example(mod=qg):
    g = golden()
    q = mod.decode_int4_packed(np.array([g["nibbles_bytes"]], np.uint8), 8)
    assert list(q[0]) == [int(v) for v in g["nibbles_values"]]
    a = bf16_bits(np.array([g["w4a16_a"]]))
    w = np.array([[0x7F, 0x18], [0x10, 0x32]], np.uint8)
    s = np.array(g["w4a16_scales"], np.float32).reshape(2, 2)
    y = mod.w4a16_gemm(a, w, s, 2)
    assert list(y[0]) == g["w4a16_y"]
    ac = np.array(g["w8a8_a_codes"], np.uint8).reshape(2, 2)
    wc = np.array(g["w8a8_w_codes"], np.uint8).reshape(1, 2)
    y = mod.w8a8_gemm(ac, np.array(g["w8a8_a_scale"], np.float32), wc, np.array(g["w8a8_w_scale"], np.float32))
    assert list(y[:, 0]) == g["w8a8_y"]
    ac = np.array([g["w4a8_a_codes"]], np.uint8)
    y = mod.w4a8_gemm(ac, np.array(g["w4a8_a_scale"], np.float32), np.array([[0x7F, 0x18], [0x10, 0x32]], np.uint8),
                      np.array(g["w4a16_scales"], np.float32).reshape(2, 2), 2)
    assert list(y[0]) == g["w4a8_y"]
    a = bf16_bits(np.array([g["w8a16_a"]]))
    wc = np.array(g["w8a16_w_codes"], np.uint8).reshape(2, 2)
    y = mod.w8a16_gemm(a, wc, np.array(g["w8a16_w_scale"], np.float32))
    assert list(y[0]) == g["w8a16_y"]


def pin_integers(mod=qg, seed=0):
    """Small integers are exact in both formats and in every partial sum: the result must equal
    integer arithmetic, times power-of-two scales, exactly."""
    rng = np.random.default_rng(seed)
    M, N, K, G = 5, 7, 64, 16
    ai = rng.integers(-4, 5, (M, K))
    wi = rng.integers(-4, 5, (N, K))
    sa = 2.0 ** rng.integers(-3, 4, M)
    sw = 2.0 ** rng.integers(-3, 4, N)
    ref = (ai @ wi.T).astype(np.float64) * sa[:, None] * sw[None, :]
    y = mod.w8a8_gemm(fp8_codes_of(ai), sa.astype(np.float32), fp8_codes_of(wi), sw.astype(np.float32))
    assert np.array_equal(y, ref)
    qi = rng.integers(-8, 8, (N, K))
    gs = 2.0 ** rng.integers(-3, 4, (N, K // G))
    ref = np.zeros((M, N))
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        ref += (ai[:, ks] @ qi[:, ks].T).astype(np.float64) * gs[None, :, g]
    y = mod.w4a16_gemm(bf16_bits(ai.astype(np.float32)), pack_int4(qi), gs.astype(np.float32), G)
    assert np.array_equal(y, ref)
    ref = (ai @ wi.T).astype(np.float64) * sw[None, :]
    y = mod.w8a16_gemm(bf16_bits(ai.astype(np.float32)), fp8_codes_of(wi), sw.astype(np.float32))
    assert np.array_equal(y, ref)
    a8 = rng.integers(-128, 128, (M, K))
    ref = np.zeros((M, N))
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        ref += (a8[:, ks] @ qi[:, ks].T).astype(np.float64) * gs[None, :, g]
    ref *= sa[:, None]
    y = mod.w4a8_gemm(a8.astype(np.int8).view(np.uint8), sa.astype(np.float32), pack_int4(qi), gs.astype(np.float32), G)
    assert np.array_equal(y, ref)


def pin_brute_force(mod=qg, seed=1):
    """A triple loop over arbitrary codes and scales, term by term, in Python floats."""
    rng = np.random.default_rng(seed)
    M, N, K, G = 3, 4, 8, 4
    tab = fp8_e4m3fn_table()
    finite = [c for c in range(256) if np.isfinite(tab[c])]
    ac = rng.choice(finite, (M, K)).astype(np.uint8)
    wc = rng.choice(finite, (N, K)).astype(np.uint8)
    sa = rng.uniform(0.01, 2, M).astype(np.float32)
    sw = rng.uniform(0.01, 2, N).astype(np.float32)
    y = mod.w8a8_gemm(ac, sa, wc, sw)
    for m, n in itertools.product(range(M), range(N)):
        ref = sum(float(tab[ac[m, k]]) * float(tab[wc[n, k]]) for k in range(K)) * float(sa[m]) * float(sw[n])
        assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    a = (rng.standard_normal((M, K))).astype(np.float32)
    ab = (a.view(np.uint32) >> 16).astype(np.uint16)            # truncation: still some bf16 value
    qi = rng.integers(-8, 8, (N, K))
    gs = rng.uniform(0.01, 1, (N, K // G)).astype(np.float32)
    y = mod.w4a16_gemm(ab, pack_int4(qi), gs, G)
    av = (ab.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for m, n in itertools.product(range(M), range(N)):
        ref = sum(av[m, k] * qi[n, k] * float(gs[n, k // G]) for k in range(K))
        assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    y = mod.w8a16_gemm(ab, wc, sw)
    for m, n in itertools.product(range(M), range(N)):
        ref = sum(av[m, k] * float(tab[wc[n, k]]) for k in range(K)) * float(sw[n])
        assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    a8 = rng.integers(0, 256, (M, K)).astype(np.uint8)            # any byte: two's complement codes
    y = mod.w4a8_gemm(a8, sa, pack_int4(qi), gs, G)
    for m, n in itertools.product(range(M), range(N)):
        ref = sum((int(a8[m, k]) - 256 * (a8[m, k] >= 128)) * qi[n, k] * float(gs[n, k // G])
                  for k in range(K)) * float(sa[m])
        assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_closed_forms(mod=qg, seed=2):
    """A = identity (codes of 1.0) with unit activation scales gives the dequantised weights;
    a constant group scale factors out of W4A16."""
    rng = np.random.default_rng(seed)
    K, N = 16, 5
    eye = fp8_codes_of(np.eye(K))
    wc = fp8_codes_of(rng.integers(-6, 7, (N, K)) * 0.5)
    sw = rng.uniform(0.5, 2, N).astype(np.float32)
    y = mod.w8a8_gemm(eye, np.ones(K, np.float32), wc, sw)
    assert np.array_equal(y, (decode_fp8_e4m3fn(wc) * sw.astype(np.float64)[:, None]).T)
    a = rng.standard_normal((3, 32)).astype(np.float32)
    ab = (a.view(np.uint32) >> 16).astype(np.uint16)
    qi = rng.integers(-8, 8, (N, 32))
    y1 = mod.w4a16_gemm(ab, pack_int4(qi), np.full((N, 4), 0.375, np.float32), 8)
    y2 = mod.w4a16_gemm(ab, pack_int4(qi), np.ones((N, 4), np.float32), 8)
    assert np.allclose(y1, 0.375 * y2, rtol=1e-14, atol=0)
    # W8A16 with A = identity (bf16 1.0) gives each channel's decoded weights times its scale
    y = mod.w8a16_gemm(bf16_bits(np.eye(K, dtype=np.float32)), wc, sw)
    assert np.array_equal(y, (decode_fp8_e4m3fn(wc) * sw.astype(np.float64)[:, None]).T)
    # and fp8-representable activations with unit activation scales agree with W8A8
    ai = rng.integers(-6, 7, (3, K)) * 0.25
    y = mod.w8a16_gemm(bf16_bits(ai.astype(np.float32)), wc, sw)
    assert np.array_equal(y, mod.w8a8_gemm(fp8_codes_of(ai), np.ones(3, np.float32), wc, sw))
    # W4A8 with unit activation scales is W4A16 on the same integers (every int8 is a bf16
    # value); a constant activation scale factors out
    a8 = rng.integers(-128, 128, (3, 32))
    gsc = rng.uniform(0.5, 2, (N, 4)).astype(np.float32)
    y1 = mod.w4a8_gemm(a8.astype(np.int8).view(np.uint8), np.ones(3, np.float32), pack_int4(qi), gsc, 8)
    y2 = mod.w4a16_gemm(bf16_bits(a8.astype(np.float32)), pack_int4(qi), gsc, 8)
    assert np.array_equal(y1, y2)
    y3 = mod.w4a8_gemm(a8.astype(np.int8).view(np.uint8), np.full(3, 0.375, np.float32), pack_int4(qi), gsc, 8)
    assert np.allclose(y3, 0.375 * y1, rtol=1e-14, atol=0)


PINS = [pin_worked_example, pin_integers, pin_brute_force, pin_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pins(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
class _Mutant:
    """The oracle module with one function replaced."""
    def __init__(self, **over):
        self.__dict__.update({k: getattr(qg, k) for k in ("decode_int4_packed", "w8a8_gemm", "w4a16_gemm",
                                                          "w8a16_gemm", "w4a8_gemm")})
        self.__dict__.update(over)


def _nibbles_swapped(packed, k):
    q = qg.decode_int4_packed(packed, k)
    out = q.copy()
    out[..., 0::2], out[..., 1::2] = q[..., 1::2], q[..., 0::2]
    return out


def _unsigned_nibbles(packed, k):
    p = np.asarray(packed, np.uint8)
    q = np.empty(p.shape[:-1] + (k,), np.int64)
    q[..., 0::2] = p & 0xF
    q[..., 1::2] = p >> 4
    return q


def _w8a8_scale_axis_swapped(a_codes, a_scale, w_codes, w_scale):
    a = decode_fp8_e4m3fn(a_codes)
    w = decode_fp8_e4m3fn(w_codes)
    y = a @ w.T
    n = min(len(a_scale), len(w_scale))
    return y * np.resize(np.asarray(w_scale, np.float64), y.shape[0])[:, None] * \
        np.resize(np.asarray(a_scale, np.float64), y.shape[1])[None, :] if n else y


def _w4a16_first_group_scale(a_bits, w_packed, w_scale, group):
    s = np.asarray(w_scale, np.float32)
    return qg.w4a16_gemm(a_bits, w_packed, np.repeat(s[:, :1], s.shape[1], axis=1), group)


def _w4a16_group_by_rows(a_bits, w_packed, w_scale, group):
    """Scales indexed as if groups ran over output rows."""
    s = np.asarray(w_scale, np.float32)
    return qg.w4a16_gemm(a_bits, w_packed, np.resize(s.T.copy(), s.shape), group)


def _w8a16_scale_by_k(a_bits, w_codes, w_scale):
    """The channel scales applied along k instead of along the output channels."""
    a = qg.decode_bf16(a_bits)
    w = decode_fp8_e4m3fn(w_codes)
    return a @ (w * np.resize(np.asarray(w_scale, np.float64), w.shape[1])[None, :]).T


def _w8a16_weights_as_bf16_bits(a_bits, w_codes, w_scale):
    """Weight codes read as the high byte of a bf16 value instead of as e4m3fn."""
    w_bits = (np.asarray(w_codes, np.uint16) << 8).astype(np.uint16)
    return qg.decode_bf16(a_bits) @ (qg.decode_bf16(w_bits) * np.asarray(w_scale, np.float64)[:, None]).T


def _w4a8_unsigned_activations(a_codes, a_scale, w_packed, w_scale, group):
    """Activation bytes read as unsigned 0..255."""
    a = np.asarray(a_codes, np.uint8).astype(np.float64) * np.asarray(a_scale, np.float64)[:, None]
    q = qg.decode_int4_packed(w_packed, a.shape[1]).astype(np.float64)
    return a @ (q * np.repeat(np.asarray(w_scale, np.float64), group, axis=1)).T


def _w4a8_scale_per_column(a_codes, a_scale, w_packed, w_scale, group):
    """The activation scales applied along the output columns."""
    y = qg.w4a8_gemm(a_codes, np.ones(len(a_scale), np.float32), w_packed, w_scale, group)
    return y * np.resize(np.asarray(a_scale, np.float64), y.shape[1])[None, :]


@pytest.mark.parametrize("mutant", [
    _Mutant(w4a8_gemm=_w4a8_unsigned_activations),
    _Mutant(w4a8_gemm=_w4a8_scale_per_column),
    _Mutant(w8a16_gemm=_w8a16_scale_by_k),
    _Mutant(w8a16_gemm=_w8a16_weights_as_bf16_bits),
    _Mutant(decode_int4_packed=_nibbles_swapped),
    _Mutant(decode_int4_packed=_unsigned_nibbles),
    _Mutant(w8a8_gemm=_w8a8_scale_axis_swapped),
    _Mutant(w4a16_gemm=_w4a16_first_group_scale),
    _Mutant(w4a16_gemm=_w4a16_group_by_rows),
], ids=["w4a8_unsigned_activations", "w4a8_scale_per_column", "w8a16_scale_along_k", "w8a16_codes_as_bf16", "nibbles_swapped", "unsigned_nibbles", "w8a8_scale_axes", "w4a16_one_group_scale", "w4a16_groups_by_rows"])
def test_planted_mistakes_fail_a_pin(mutant):
    # the W4A16 mutants call the real decoder; make them use the mutant's too where it differs
    failed = 0
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1
