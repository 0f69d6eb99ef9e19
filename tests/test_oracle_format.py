"""Pins of the oracle's NVFP4 format functions against things other than itself:
the format's closed form, torch's float8_e4m3fn codec (a library routine),
exact-rational brute force, and the byte figures the pages print."""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # 1 sign, 2 exponent (bias 1), 1 mantissa bit


def torch_e4m3_decode(byte: int) -> float:
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def torch_e4m3_rne(q: float) -> int:
    """Library RNE conversion of an fp32-exact value to E4M3 (no saturation)."""
    return int(torch.tensor([q], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


E4M3_FINITE = [Fraction(torch_e4m3_decode(b)) for b in range(127)]  # bytes 0x00..0x7E, increasing


def brute_scale(amax: float, g: float = 1.0) -> int:
    """Nearest non-negative finite E4M3 to the exact amax / (6 g); ties to the even byte."""
    q = Fraction(amax) / (6 * Fraction(g))
    best, bd = None, None
    for k, v in enumerate(E4M3_FINITE):
        d = abs(q - v)
        if bd is None or d < bd or (d == bd and k % 2 == 0):
            best, bd = k, d
    return best


def brute_code(x: float, D: Fraction) -> int:
    sign = 8 if math.copysign(1.0, x) < 0 else 0
    if D == 0:
        return sign
    q = abs(Fraction(x)) / D
    best, bd = None, None
    for k, v in enumerate(E2M1_MAGNITUDES):
        d = abs(q - Fraction(v))
        if bd is None or d < bd or (d == bd and k % 2 == 0):
            best, bd = k, d
    return sign | best


# ---- decode --------------------------------------------------------------------
def test_e2m1_closed_form(oracle_lib):
    for c in range(16):
        v = oracle_lib.e2m1_value(c)
        want = E2M1_MAGNITUDES[c & 7]
        assert abs(v) == want
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)  # 0x8 is -0


def test_e2m1_through_library_e4m3(oracle_lib):
    """Re-encode each E2M1 code's fields as an E4M3 byte (exponent re-biased 1 -> 7,
    mantissa bit moved to the top of the 3-bit field) and decode it with torch."""
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            byte = 0
        elif e == 0:  # subnormal 0.5 = 2^-1
            byte = (6 << 3)
        else:
            byte = ((e + 6) << 3) | (m << 2)
        byte |= s << 7
        assert oracle_lib.e2m1_value(c) == torch_e4m3_decode(byte)


def test_e4m3_decode_all_bytes_vs_library(oracle_lib):
    for b in range(256):
        v, w = oracle_lib.e4m3_value(b), torch_e4m3_decode(b)
        if math.isnan(w):
            assert math.isnan(v), b
        else:
            assert v == w and math.copysign(1, v) == math.copysign(1, w), b
    assert oracle_lib.e4m3_value(0x01) == 2.0 ** -9
    assert oracle_lib.e4m3_value(0x08) == 2.0 ** -6
    assert oracle_lib.e4m3_value(0x7E) == 448.0
    assert math.isnan(oracle_lib.e4m3_value(0x7F)) and math.isnan(oracle_lib.e4m3_value(0xFF))


# ---- block scale -----------------------------------------------------------------
def _scale_probe_points():
    pts = set()
    vals = [float(v) for v in E4M3_FINITE]
    for k in range(126):
        mid = (vals[k] + vals[k + 1]) / 2
        pts.update([vals[k], mid, float(np.nextafter(np.float32(mid), np.float32(0))),
                    float(np.nextafter(np.float32(mid), np.float32(1e9)))])
    rng = random.Random(3)
    for _ in range(3000):
        e = rng.uniform(-12, 9)
        pts.add(float(np.float32(2.0 ** e)))
    return sorted(p for p in pts if p <= 448.0)


def test_scale_byte_vs_library_rne(oracle_lib):
    """For q with <= 22 significant bits, amax = 6q is exact in fp32 and the oracle's
    E4M3(amax/6) must equal torch's RNE conversion of q."""
    n = 0
    for q in _scale_probe_points():
        m, e = math.frexp(q)
        if q != 0 and (m * 2 ** 22) != int(m * 2 ** 22):
            continue
        amax = float(np.float32(6.0 * q))
        assert amax == 6.0 * q
        assert oracle_lib.scale_byte(amax) == torch_e4m3_rne(q), q
        n += 1
    assert n > 1000


def test_scale_byte_saturates(oracle_lib):
    for amax in [6 * 448.0, 6 * 460.0, 6 * 464.0, 6 * 1000.0, 3.0e38]:
        assert oracle_lib.scale_byte(amax) == 0x7E


def test_scale_byte_bruteforce(oracle_lib):
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        np.float32(2.0) ** rng.uniform(-14, 12, 4000).astype(np.float32),
        rng.standard_normal(1000).astype(np.float32) * 3,
    ])
    for a in np.abs(xs).astype(np.float32):
        assert oracle_lib.scale_byte(float(a)) == brute_scale(float(a)), float(a)


def test_scale_byte_power_of_two_global_scale(oracle_lib):
    rng = np.random.default_rng(12)
    for g in [0.25, 0.5, 2.0, 8.0]:
        for a in np.abs(rng.standard_normal(300).astype(np.float32)) * 4:
            assert oracle_lib.scale_byte(float(a), g) == brute_scale(float(a), g)


# ---- element codes ------------------------------------------------------------------
def test_e2m1_code_bruteforce(oracle_lib):
    rng = np.random.default_rng(13)
    for _ in range(6000):
        s = int(rng.integers(0, 127))
        D = E4M3_FINITE[s]
        x = float(np.float32(rng.standard_normal() * float(D) * rng.uniform(0, 8)))
        assert oracle_lib.e2m1_code(x, float(D)) == brute_code(x, D), (x, s)


def test_e2m1_code_threshold_edges(oracle_lib):
    """Every E2M1 midpoint, for every scale, exactly and one fp32 ulp either side."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    n = 0
    for s in range(1, 127):
        D = E4M3_FINITE[s]
        for m in mids:
            t = np.float32(m * float(D))
            assert Fraction(float(t)) == Fraction(m) * D
            for x in (t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e9))):
                for sgn in (1, -1):
                    xv = float(np.float32(sgn * x))
                    assert oracle_lib.e2m1_code(xv, float(D)) == brute_code(xv, D), (xv, s)
                    n += 1
    assert n > 5000
    # the tie table: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4 (code indices
    # of 0, 0.5, 1, 1.5, 2, 3, 4, 6 are 0..7), values above 6 saturate to 6
    for m, want in zip(mids, [0, 2, 2, 4, 4, 6, 6]):
        assert oracle_lib.e2m1_code(m, 1.0) == want
    assert oracle_lib.e2m1_code(100.0, 1.0) == 7
    assert oracle_lib.e2m1_code(-0.0, 1.0) == 8
    assert oracle_lib.e2m1_code(-0.1, 1.0) == 8


# ---- whole blocks -----------------------------------------------------------------
def test_worked_example_block_of_ones(oracle_lib):
    # amax = 1: 1/6 lies between 0.15625 (0x22) and 0.171875 (0x23), nearer the latter
    codes, s = oracle_lib.quantize_block16([1.0] * 16)
    assert s == 0x23 and oracle_lib.e4m3_value(s) == 0.171875
    assert list(codes) == [0x77] * 8  # code 7 = 6.0 in both nibbles
    assert 6 * 0.171875 == 1.03125  # so sixteen 1.0 values dequantize to 1.03125 each


def _dequant_block(oracle_lib, codes, s, g=1.0):
    out = []
    for b in codes:
        out += [oracle_lib.e2m1_value(int(b) & 15), oracle_lib.e2m1_value(int(b) >> 4)]
    return np.array(out) * oracle_lib.e4m3_value(s) * g


def test_round_trip_of_representable_blocks(oracle_lib):
    rng = np.random.default_rng(14)
    for _ in range(800):
        s = int(rng.integers(8, 127))  # normal scales
        c = rng.integers(0, 16, 16)
        c[rng.integers(0, 16)] = 7 | (8 * int(rng.integers(0, 2)))  # the block's max magnitude is 6
        x = np.array([oracle_lib.e2m1_value(int(ci)) for ci in c]) * oracle_lib.e4m3_value(s)
        codes, s2 = oracle_lib.quantize_block16(x.astype(np.float32))
        assert s2 == s
        got = []
        for b in codes:
            got += [int(b) & 15, int(b) >> 4]
        assert got == [int(ci) for ci in c]


def test_idempotence_normal_scales_and_error_bound(oracle_lib):
    rng = np.random.default_rng(15)
    normal = 0
    for _ in range(3000):
        x = (rng.standard_normal(16) * np.exp(rng.uniform(-3, 3))).astype(np.float32)
        codes, s = oracle_lib.quantize_block16(x)
        D = oracle_lib.e4m3_value(s)
        xh = _dequant_block(oracle_lib, codes, s)
        if s >= 0x08:
            normal += 1
            assert np.all(np.abs(x - xh) <= D)  # error at most one scale step
            codes2, s2 = oracle_lib.quantize_block16(xh.astype(np.float32))
            assert s2 == s and list(codes2) == list(codes)
    assert normal > 2500


def test_zero_scale_reading(oracle_lib):
    x = np.array([1e-5, -2e-5] * 8, dtype=np.float32)  # amax/6 < 2^-10: scale rounds to 0
    codes, s = oracle_lib.quantize_block16(x)
    assert s == 0
    assert list(codes) == [0x80] * 8  # magnitude 0, sign of x kept


def test_non_finite_reading(oracle_lib):
    """Reading for non-finite inputs (the pages are silent): a NaN element is left
    out of the block's amax and encodes as magnitude 0 with its sign bit; an
    infinity saturates the block scale at 448 and encodes as magnitude 6. The
    finite elements are encoded against the scale that results, per the brute
    force of every candidate code."""
    rng = np.random.default_rng(5)
    for sign in (1.0, -1.0):
        for pos in (3, 15):  # the NaN after the largest value, and last
            x = rng.standard_normal(16).astype(np.float32)
            x[0] = np.float32(4.0)  # the block's largest magnitude comes first
            x[pos] = np.float32(math.copysign(math.nan, sign))
            codes, s = oracle_lib.quantize_block16(x)
            finite = np.delete(x, pos)
            assert s == brute_scale(float(np.abs(finite).max()))
            D = E4M3_FINITE[s]
            nib = [(codes[i // 2] >> (4 * (i % 2))) & 15 for i in range(16)]
            assert nib[pos] == (8 if sign < 0 else 0)
            assert all(nib[i] == brute_code(float(x[i]), D) for i in range(16) if i != pos)
            x[pos] = np.float32(sign * math.inf)
            codes, s = oracle_lib.quantize_block16(x)
            assert s == 0x7E
            nib = [(codes[i // 2] >> (4 * (i % 2))) & 15 for i in range(16)]
            assert nib[pos] == (15 if sign < 0 else 7)
            assert all(nib[i] == brute_code(float(x[i]), E4M3_FINITE[0x7E]) for i in range(16) if i != pos)
    # an all-NaN block: amax 0, scale 0, every code magnitude 0 with its sign
    codes, s = oracle_lib.quantize_block16(np.array([math.nan, -math.nan] * 8, dtype=np.float32))
    assert s == 0 and list(codes) == [0x80] * 8


def test_global_scale_power_of_two(oracle_lib):
    rng = np.random.default_rng(16)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        c1, s1 = oracle_lib.quantize_block16(x, 1.0)
        c2, s2 = oracle_lib.quantize_block16((x * 4).astype(np.float32), 4.0)
        assert s1 == s2 and list(c1) == list(c2)
        assert np.array_equal(_dequant_block(oracle_lib, c2, s2, 4.0), 4 * _dequant_block(oracle_lib, c1, s1))


# ---- byte accounting (figures printed on the pages) -------------------------------------
def test_byte_accounting_against_page_figures(oracle_lib):
    with open(os.path.join(HERE, "golden", "byte_accounting.json")) as f:
        gold = json.load(f)
    blk = gold["block_bytes"]
    ratio = (blk["packed_bytes"] + blk["scale_bytes"]) / blk["fp8_bytes"]
    assert ratio == gold["ratio_to_fp8"]["value"]
    assert round(100 * ratio) == gold["ratio_percent_approx"]["value"]
    assert round(1 / ratio, 2) == gold["idealised_capacity_gain"]["value"]
    # the oracle's pool: one page of one KV head holds 16 tokens x (K, V) x 128 values
    pool_ratio = oracle_lib.pool_bytes(1, 1) / (16 * 2 * 128)
    assert pool_ratio == ratio
    ll = gold["llama33_70b_values_per_token"]
    vpt = 2 * ll["layers"] * ll["kv_heads"] * ll["head_dim"]
    assert vpt == ll["value"]
    gib = 2.0 ** 30
    c128 = gold["llama33_70b_128k_conversation_gib"]
    assert vpt * c128["tokens"] * 1 / gib == c128["fp8"]
    assert vpt * c128["tokens"] * pool_ratio / gib == c128["nvfp4"]
    s8 = gold["llama33_70b_8k_sessions"]
    assert vpt * s8["tokens"] / gib == s8["fp8_gib"]
    assert round(vpt * s8["tokens"] * pool_ratio / gib, 2) == s8["nvfp4_gib"]
    assert round(s8["usable_fraction"] * s8["card_gib"] - s8["reserve_gib"], 1) == s8["budget_gib"]
    free = s8["budget_gib"] - s8["fp8_weights_gib"]
    assert round(free, 1) == c128["free_next_to_fp8_weights"]
    assert int(free / s8["fp8_gib"]) == s8["sessions_fp8"]
    assert int(free / (vpt * s8["tokens"] * pool_ratio / gib)) == s8["sessions_nvfp4"]
    # per token and layer of the 8-KV-head, head-dim-128 geometry: 1152 bytes
    assert oracle_lib.pool_bytes(1, 8) // 16 == 1152


def test_fp8_workspace_rounding_vs_library(oracle_lib):
    # the FP8 E4M3 workspace code of a value: below 448 it is the library's
    # round-to-nearest-even float8_e4m3fn cast; above, saturation to +-448
    rng = np.random.default_rng(31)
    # float32 inputs (ties and their float32 neighbours are exact there), so the
    # library rounds once, from the same value the oracle sees
    finite = np.array([oracle_lib.e4m3_value(b) for b in range(127)], dtype=np.float32)
    mids = (0.5 * (finite[:-1].astype(np.float64) + finite[1:])).astype(np.float32)  # exact ties
    xs = np.concatenate([finite, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                         rng.uniform(0, 448, 2000).astype(np.float32),
                         rng.uniform(0, 2.0 ** -6, 500).astype(np.float32), np.zeros(1, np.float32)])
    xs = xs[xs < 448]
    for sgn in (np.float32(1.0), np.float32(-1.0)):
        v = sgn * xs
        lib_codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ours = oracle_lib.e4m3_codes_of(v)
        assert np.array_equal(ours, lib_codes), (v[ours != lib_codes][:5], ours[ours != lib_codes][:5])
    for x, want in [(448.0, 0x7E), (464.0, 0x7E), (2688.0, 0x7E), (-1e30, 0xFE), (-0.0, 0x80), (0.0, 0x00),
                    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -9 * 7.5, 0x08)]:
        assert oracle_lib.e4m3_code_of(x) == want, (x, want)


# ---- any finite global scale g (not only powers of two) -------------------------------
# g values with many significant bits (0.3, 1/2688 as binary32), few bits but not a
# power of two (7.5, 0.75: their thresholds are exact in binary32, so exact ties
# occur), and a random one.
NON_POW2_G = [float(np.float32(0.3)), float(np.float32(1 / 2688)), 7.5, 0.75, float(np.float32(1.8472671))]


def _f32_near(q: Fraction) -> list:
    """The binary32 nearest to q and its two neighbours (all positive)."""
    t = np.float32(float(q))
    return [float(t), float(np.nextafter(t, np.float32(0))), float(np.nextafter(t, np.float32(np.inf)))]


def test_scale_byte_non_power_of_two_global_scale(oracle_lib):
    rng = np.random.default_rng(17)
    n_ties = 0
    for g in NON_POW2_G:
        G = Fraction(g)
        # every E4M3 midpoint times 6 g, as the nearest binary32 and one ulp either side
        for k in range(126):
            mid = (E4M3_FINITE[k] + E4M3_FINITE[k + 1]) / 2
            for a in _f32_near(mid * 6 * G):
                n_ties += Fraction(a) == mid * 6 * G
                assert oracle_lib.scale_byte(a, g) == brute_scale(a, g), (a, g, k)
        for a in (np.abs(rng.standard_normal(200)) * 6 * g * np.exp(rng.uniform(-8, 6, 200))).astype(np.float32):
            assert oracle_lib.scale_byte(float(a), g) == brute_scale(float(a), g), (float(a), g)
    assert n_ties > 200  # the few-bit g produce exact ties, decided to the even byte


def test_e2m1_code_non_power_of_two_divisor(oracle_lib):
    """Codes against D = E4M3(s) g (exact in double: at most 28 significant bits) at
    every E2M1 midpoint times D, as the nearest binary32 and one ulp either side."""
    mids = [Fraction(m) for m in ("1/4", "3/4", "5/4", "7/4", "5/2", "7/2", "5")]
    n = 0
    for g in NON_POW2_G:
        for s in range(1, 127, 3):
            D = E4M3_FINITE[s] * Fraction(g)
            assert Fraction(float(D)) == D
            for m in mids:
                for a in _f32_near(m * D):
                    for xv in (a, -a):
                        assert oracle_lib.e2m1_code(xv, float(D)) == brute_code(xv, D), (xv, s, g)
                        n += 1
    assert n > 8000


def _nibbles(codes):
    return [(int(codes[i // 2]) >> (4 * (i % 2))) & 15 for i in range(16)]


def test_quantize_block_non_power_of_two_global_scale(oracle_lib):
    rng = np.random.default_rng(18)
    mids = [Fraction(m) for m in ("1/4", "3/4", "5/4", "7/4", "5/2", "7/2", "5")]
    for g in NON_POW2_G:
        # blocks whose values sit on the code thresholds of their own scale (+-1 ulp)
        for s_want in (9, 40, 77, 110):
            D = E4M3_FINITE[s_want] * Fraction(g)
            top = np.float32(float(6 * D))  # amax near 6 D: the scale is s_want or a neighbour
            s = brute_scale(float(top), g)
            D = E4M3_FINITE[s] * Fraction(g)
            vals = [v for m in mids for v in _f32_near(m * D)][:15]
            x = np.array([float(top)] + [v if i % 2 else -v for i, v in enumerate(vals)], dtype=np.float32)
            codes, s2 = oracle_lib.quantize_block16(x, g)
            assert s2 == s
            assert _nibbles(codes) == [brute_code(float(v), D) for v in x], (g, s)
        for _ in range(150):
            x = (rng.standard_normal(16) * g * np.exp(rng.uniform(-4, 6))).astype(np.float32)
            codes, s = oracle_lib.quantize_block16(x, g)
            assert s == brute_scale(float(np.abs(x).max()), g)
            D = E4M3_FINITE[s] * Fraction(g)
            assert _nibbles(codes) == [brute_code(float(v), D) for v in x]


def test_dequant_values_are_exact_products_for_any_g(oracle_lib):
    """x^ = E2M1(c) E4M3(s) g exactly (at most 30 significant bits, exact in double)."""
    rng = np.random.default_rng(19)
    for g in NON_POW2_G:
        k = (rng.standard_normal((3, 2, 128)) * g * 4).astype(np.float32)
        pool = oracle_lib.quantize_to_pool(k, -k, np.array([16 * 2 + 5, 3, 16 + 15], dtype=np.int32), 3, g=g)
        for t, slot in enumerate((37, 3, 31)):
            for h in range(2):
                for kind in (0, 1):
                    row = oracle_lib.dequant_row(pool, slot // 16, slot % 16, h, kind, 2, g)
                    slab = pool[oracle_lib.slab_offset(slot // 16, h, kind, 2):][:1152]
                    for d in range(0, 128, 7):
                        nib = oracle_lib.code_nibble(kind, slot % 16, d)
                        c = (int(slab[nib // 2]) >> (4 * (nib % 2))) & 15
                        sb = int(slab[oracle_lib.scale_byte_offset(kind, slot % 16, d // 16)])
                        want = Fraction(E2M1_MAGNITUDES[c & 7]) * (-1 if c & 8 else 1) * E4M3_FINITE[sb] * Fraction(g)
                        assert Fraction(row[d]) == want, (g, t, h, kind, d)


def _bf16_nearest_even(x: float) -> int:
    """Exact-rational nearest bf16 (8 significant bits), ties to the even significand."""
    q = abs(Fraction(x))
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    if q == 0:
        return sign
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    ulp = Fraction(2) ** (e - 7)
    lo = (q // ulp)
    r = q - lo * ulp
    n = lo + (1 if (r > ulp / 2 or (r == ulp / 2 and lo % 2 == 1)) else 0)
    v = float(n * ulp)
    return sign | int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)[0]) & 0x7FFF


def test_bf16_rounding_of_exact_values(oracle_lib):
    rng = np.random.default_rng(20)
    # float32-exact inputs: the library's float32 -> bf16 cast rounds once, to nearest even
    f = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 100,
                        (1 + np.arange(256, dtype=np.float32) / 256) * np.float32(3.0)])
    lib = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_lib.bf16_bits_of(f.astype(np.float64)), lib)
    # doubles with more bits than binary32 (dequantized products at non-power-of-two g),
    # and exact ties with a tiny excess either side
    xs = [float(Fraction(c) * E4M3_FINITE[s] * Fraction(g)) for g in NON_POW2_G for s in range(1, 127, 5)
          for c in ("1/2", "3/2", "3", "6")]
    xs += [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8 - 2.0 ** -40, -(1 + 2.0 ** -8)]
    got = oracle_lib.bf16_bits_of(np.array(xs))
    assert [int(v) for v in got] == [_bf16_nearest_even(x) for x in xs]
    assert [int(v) for v in got[-5:]] == [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80]
