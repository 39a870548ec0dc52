"""Pins of the oracle's value tables, packers and roundings (CPU only).

Each test ties an oracle function to something outside itself: a published
value table (fixtures under tests/golden/, each with its source), a closed form
from a published construction, the worked examples printed on the pages, exact
rational arithmetic, brute force, or an independent library conversion.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import pack as P
from conftest import read_golden


# ----------------------------------------------------------------------------- NF4 table
def test_nf4_table_matches_published_values():
    vals = np.array([float(v) for v in read_golden("nf4_qlora.txt")], dtype=np.float32)
    assert vals.shape == (16,)
    assert np.array_equal(vals.view(np.uint32), oracle.NF4_TABLE_F32.view(np.uint32))


def test_nf4_table_matches_closed_form_quantiles():
    cf = oracle.nf4_table_closed_form()
    assert np.max(np.abs(cf - oracle.NF4_TABLE_F32.astype(np.float64))) < 2e-7


def test_nf4_table_invariants():
    t = oracle.NF4_TABLE_F32
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert t[0] == -1.0 and t[15] == 1.0
    assert t.view(np.uint32)[7] == 0          # +0.0 exactly
    assert (t < 0).sum() == 7 and (t > 0).sum() == 8


# ----------------------------------------------------------------------------- e2m1 / e8m0
def test_e2m1_matches_ocp_table():
    rows = [r.split() for r in read_golden("e2m1_ocp.txt")]
    for code, val in rows:
        got = oracle.e2m1_value(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code
    assert np.array_equal(oracle.E2M1_TABLE, np.array([float(v) for _, v in rows]))
    assert math.copysign(1.0, oracle.E2M1_TABLE[8]) == -1.0   # -0.0 keeps its sign


def test_e8m0_all_bytes():
    x = np.arange(256)
    v = oracle.e8m0_value(x)
    for b in range(255):
        assert v[b] == math.ldexp(1.0, b - 127)
    assert math.isnan(v[255])


# ----------------------------------------------------------------------------- nibble order
def test_nibble_order_convention():
    # NF4: element 2j in the high nibble; MXFP4: element 2j in the low nibble.
    assert P.pack_nf4_codes(np.array([1, 2], np.uint8))[0] == 0x12
    assert P.pack_mxfp4_codes(np.array([1, 2], np.uint8))[0] == 0x21
    assert list(P.unpack_nf4_codes(np.array([0xAB], np.uint8))) == [0xA, 0xB]
    assert list(P.unpack_mxfp4_codes(np.array([0xAB], np.uint8))) == [0xB, 0xA]


# ----------------------------------------------------------------------------- page examples
def _page():
    d = {}
    for r in read_golden("page_cpu_examples.txt"):
        k, v = [s.strip() for s in r.split("=")]
        d[k] = v
    return d


def _shape(s):
    return tuple(int(x) for x in s.split())


def test_nf4_page_round_trip():
    page = _page()
    rng = np.random.default_rng(1234)
    w = rng.standard_normal(_shape(page["nf4.input_shape"])).astype(np.float32)
    q, s = oracle.quantize_pack_nf4(w)
    assert q.shape == _shape(page["nf4.codes_shape"]) and q.dtype == np.uint8
    assert s.shape == _shape(page["nf4.absmax_shape"]) and s.dtype == np.float32
    wq = oracle.nf4_w32(q, s)
    rel = np.linalg.norm(wq - w) / np.linalg.norm(w)
    assert abs(rel - float(page["nf4.rel_err_approx"])) < 0.006, rel
    q2, s2 = oracle.quantize_pack_nf4(wq)
    assert page["nf4.repack_idempotent"] == "True"
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_mxfp4_page_round_trip():
    page = _page()
    rng = np.random.default_rng(4321)
    w = rng.standard_normal(_shape(page["mxfp4.input_shape"])).astype(np.float32)
    b, s = oracle.quantize_pack_mxfp4(w)
    assert b.shape == _shape(page["mxfp4.blocks_shape"]) and b.dtype == np.uint8
    assert s.shape == _shape(page["mxfp4.scales_shape"]) and s.dtype == np.uint8
    wq = oracle.dequant_mxfp4(b, s)
    rel = np.linalg.norm(wq - w) / np.linalg.norm(w)
    assert abs(rel - float(page["mxfp4.rel_err_approx"])) < 0.01, rel
    # quantiser outputs re-quantise to the same bytes
    b2, s2 = oracle.quantize_pack_mxfp4(wq.astype(np.float32))
    assert np.array_equal(b2, b) and np.array_equal(s2, s)


def test_nf4_refuses_non_2d():
    with pytest.raises(ValueError):
        oracle.quantize_pack_nf4(np.zeros((2, 2, 64), np.float32))


# ----------------------------------------------------------------------------- quantisers, brute force
def test_nf4_quantiser_is_nearest_code_brute_force():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((4, 128)).astype(np.float32)
    w[1, 64:] = 0.0                                  # an all-zero block
    q, s = oracle.quantize_pack_nf4(w)
    codes = P.unpack_nf4_codes(q)
    T = [Fraction(float(t)) for t in oracle.NF4_TABLE_F32]
    for n in range(4):
        for k in range(128):
            am = Fraction(float(s[n, k // 64]))
            assert float(am) == float(np.max(np.abs(w[n, (k // 64) * 64:(k // 64 + 1) * 64])))
            x = Fraction(float(w[n, k])) / am if am else Fraction(0)
            dist = [abs(x - t) for t in T]
            best = min(range(16), key=lambda i: (dist[i], i))   # ties -> lower code
            assert codes[n, k] == best, (n, k)
    assert np.all(codes[1, 64:] == 7) and s[1, 1] == 0.0


def test_mxfp4_quantiser_brute_force():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((3, 64)) * 3).astype(np.float32)
    b, s = oracle.quantize_pack_mxfp4(w)
    codes = P.unpack_mxfp4_codes(b.reshape(3, 32))
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for n in range(3):
        for k in range(64):
            blk = w[n, (k // 32) * 32:(k // 32 + 1) * 32].astype(np.float64)
            amax = np.abs(blk).max()
            X = math.floor(math.log2(amax)) - 2
            assert s[n, k // 32] == X + 127
            v = float(w[n, k]) / 2.0 ** X
            a = min(abs(v), 6.0)
            best = min(range(8), key=lambda i: (abs(a - mags[i]), i % 2, i))  # ties -> even
            assert codes[n, k] & 7 == best, (n, k, v)
            assert (codes[n, k] >> 3) == (1 if math.copysign(1.0, v) < 0 else 0)


# ----------------------------------------------------------------------------- exact products
def test_nf4_fp64_product_is_exact_and_w32_is_its_rounding():
    rng = np.random.default_rng(9)
    q = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    s = (rng.standard_normal((8, 2)) * 0.05).astype(np.float32)
    w64 = oracle.dequant_nf4(q, s)
    w32 = oracle.nf4_w32(q, s)
    codes = P.unpack_nf4_codes(q)
    for n in range(8):
        for k in range(0, 128, 7):
            exact = Fraction(float(oracle.NF4_TABLE_F32[codes[n, k]])) * Fraction(float(s[n, k // 64]))
            assert Fraction(w64[n, k]) == exact
            # fp32 rounding of the exact product: nearest float32, ties to even
            f = np.float32(float(exact))
            assert w32[n, k] == f


def test_mxfp4_specials():
    # code 8 is -0.0, e8m0 0 and 1 give fp32 subnormals, >= 253 overflow, 255 NaN
    codes = np.array([[0x08, 0x71, 0x00, 0x00] * 4], np.uint8)      # 16 bytes = 32 codes
    for sb, check in [(127, "neg0"), (0, "sub"), (1, "sub"), (254, "inf"), (255, "nan")]:
        w = oracle.mxfp4_w32(codes, np.array([[sb]], np.uint8))
        if check == "neg0":
            assert w[0, 0] == 0.0 and np.signbit(w[0, 0])       # element 0 = low nibble of 0x08
        elif check == "sub":
            # element 2 = low nibble of 0x71 = code 1 (0.5) -> 0.5 * 2^(sb-127)
            assert w[0, 2] == np.float32(math.ldexp(0.5, sb - 127)) and w[0, 2] != 0
            assert abs(w[0, 2]) < np.finfo(np.float32).tiny
        elif check == "inf":
            assert np.isinf(w[0, 3])                             # code 7 = 6.0 * 2^127
        else:
            assert np.all(np.isnan(w))


# ----------------------------------------------------------------------------- roundings
def test_bf16_rne_known_vectors():
    f = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, np.inf, -np.inf,
                  np.finfo(np.float32).max], dtype=np.float32)
    assert list(P.bf16_rne_bits(f)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F80, 0xFF80, 0x7F80]
    nan = np.array([np.nan], np.float32)
    b = P.bf16_rne_bits(nan)[0]
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(10)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    mine = P.bf16_rne_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_fp16_rne_matches_torch_conversion():
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(100000) * 10.0 ** rng.integers(-9, 6, 100000)).astype(np.float32)
    mine = P.fp16_rne_bits(f)
    ref = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert P.fp16_rne_bits(np.array([1 + 2 ** -11], np.float32))[0] == 0x3C00   # tie -> even
