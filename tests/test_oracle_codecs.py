"""Pins for the oracle's number-format decoders (CPU only).

Each check compares the oracle's closed-form decoder with something independent of
it: a value table transcribed from the format's published specification (E2M1), a
library routine (math.ldexp for E8M0, numpy.float16 for binary16, torch's
float32 -> bfloat16 conversion for rounding), or constructed midpoints.
"""
import math
import os

import numpy as np
import pytest

from oracle import codecs


def _load_e2m1_table(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "e2m1_table.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def test_e2m1_exhaustive_against_spec_table(golden_dir):
    table = _load_e2m1_table(golden_dir)
    assert sorted(table) == list(range(16))
    for c in range(16):
        got = codecs.e2m1_value(c)
        assert got == table[c], c
        assert math.copysign(1.0, got) == math.copysign(1.0, table[c]), c  # -0 for code 8
    arr = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(arr, np.array([table[c] for c in range(16)]))
    assert np.signbit(arr[8])


def test_e8m0_all_codes_against_ldexp():
    for b in range(255):
        assert codecs.e8m0_value(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(codecs.e8m0_value(255))
    arr = codecs.e8m0_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(arr[:255], np.ldexp(1.0, np.arange(255) - 127))


def test_fp16_all_65536_codes_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = codecs.fp16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # scalar form agrees with the array form
    for b in (0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00, 0x8001, 0xFBFF):
        assert codecs.fp16_value(b) == got[b]


def test_bf16_decode_all_codes_against_float32_upper_half():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = codecs.bf16_decode(bits.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    for b in (0x0001, 0x007F, 0x0080, 0x3F80, 0x7F7F, 0x7F80, 0xBF80):
        assert codecs.bf16_value(b) == got[b]


def test_bf16_round_trip_identity_on_all_finite_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_decode(bits)
    fin = np.isfinite(v)
    r = codecs.bf16_round(v[fin])
    assert np.array_equal(r, v[fin])
    b = codecs.bf16_bits(r)
    # -0 and +0 both round-trip to themselves
    assert np.array_equal(b, bits[fin])


def test_bf16_round_constructed_midpoints_tie_to_even():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    # exactly halfway between 1 and 1+ulp: 1 has an even mantissa -> stays 1
    assert codecs.bf16_round(np.array([one + ulp / 2]))[0] == one
    # halfway between 1+ulp (odd) and 1+2ulp (even) -> goes up
    assert codecs.bf16_round(np.array([one + 1.5 * ulp]))[0] == one + 2 * ulp
    # a hair above/below the midpoint decides by distance
    assert codecs.bf16_round(np.array([one + ulp / 2 + 2.0 ** -40]))[0] == one + ulp
    assert codecs.bf16_round(np.array([one + 1.5 * ulp - 2.0 ** -40]))[0] == one + ulp
    # negative side mirrors
    assert codecs.bf16_round(np.array([-(one + 1.5 * ulp)]))[0] == -(one + 2 * ulp)
    # carry into the next binade
    assert codecs.bf16_round(np.array([2.0 - ulp / 4]))[0] == 2.0
    # subnormal spacing 2^-133, tie to even
    s = 2.0 ** -133
    assert codecs.bf16_round(np.array([2.5 * s]))[0] == 2 * s
    assert codecs.bf16_round(np.array([3.5 * s]))[0] == 4 * s
    # overflow
    big = 2.0 ** 127 * (2.0 - 2.0 ** -7)
    assert codecs.bf16_round(np.array([big]))[0] == big
    mid = 2.0 ** 128 - 2.0 ** 119            # halfway from big to 2^128; big is odd -> up
    assert codecs.bf16_round(np.array([mid]))[0] == np.inf
    assert codecs.bf16_round(np.array([-mid]))[0] == -np.inf
    assert codecs.bf16_round(np.array([mid - 2.0 ** 80]))[0] == big


def test_bf16_round_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    # fp32 inputs are exact in fp64, so torch's single fp32 -> bf16 RNE step and the
    # oracle's fp64 -> bf16 step must agree bit for bit.
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # also every exact midpoint pattern (low half 0x8000) and neighbours
    hi = rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32)
    mids = np.concatenate([(hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    fm = mids.astype(np.uint32).view(np.float32)
    f = np.concatenate([f, fm[np.isfinite(fm)]])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_bits(codecs.bf16_round(f.astype(np.float64)))
    assert np.array_equal(got, ref)


def test_mxfp4_nibble_order_fixture(golden_dir):
    with open(os.path.join(golden_dir, "mxfp4_nibble_order.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    d = {r[0]: r[1:] for r in rows}
    codes = np.array([int(b, 16) for b in d["bytes"]], dtype=np.uint8)[None, :]
    want = np.array([float(v) for v in d["values"]])
    got = codecs.dequant_mxfp4(codes, np.array([[127]], dtype=np.uint8))[0]
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_mxfp4_block_scale_applies_per_32_elements(golden_dir):
    table = _load_e2m1_table(golden_dir)
    rng = np.random.default_rng(1)
    rows, K = 3, 96
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(rows, K // 32), dtype=np.uint8)
    got = codecs.dequant_mxfp4(codes, scales)
    for r in range(rows):
        for i in range(K):
            byte = int(codes[r, i // 2])
            c = (byte >> 4) if (i % 2) else (byte & 0xF)
            want = table[c] * math.ldexp(1.0, int(scales[r, i // 32]) - 127)
            assert got[r, i] == want


def test_q8_0_block_scale_applies_per_32_elements():
    rng = np.random.default_rng(2)
    rows, K = 3, 96
    q = rng.integers(-128, 128, size=(rows, K), dtype=np.int8)
    d = rng.uniform(-1, 1, size=(rows, K // 32)).astype(np.float16).view(np.uint16)
    got = codecs.dequant_q8_0(q, d)
    dv = d.view(np.float16).astype(np.float64)
    for r in range(rows):
        for i in range(K):
            assert got[r, i] == float(q[r, i]) * dv[r, i // 32]


def _q4_k_plane(sc, m, d_bits, dmin_bits):
    """Scale plane bytes written out field by field with struct (independent of numpy views)."""
    import struct
    rows, nb = sc.shape
    ns = nb // 8
    out = np.zeros((rows, 2 * nb + 4 * ns), dtype=np.uint8)
    for r in range(rows):
        raw = bytearray()
        for b in range(nb):
            raw += bytes([int(sc[r, b]), int(m[r, b])])
        for s in range(ns):
            raw += struct.pack("<HH", int(d_bits[r, s]), int(dmin_bits[r, s]))
        out[r] = np.frombuffer(bytes(raw), dtype=np.uint8)
    return out


def test_q4_k_brute_force_per_element():
    """Every element against d*sc*q - dmin*m evaluated with Python floats, the codes read
    nibble by nibble and the fp16 fields decoded by struct's IEEE half format."""
    import struct
    rng = np.random.default_rng(3)
    rows, K = 3, 512
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(rows, K // 32))
    m = rng.integers(0, 64, size=(rows, K // 32))
    d_bits = rng.uniform(-1, 1, size=(rows, K // 256)).astype(np.float16).view(np.uint16)
    dmin_bits = rng.uniform(-1, 1, size=(rows, K // 256)).astype(np.float16).view(np.uint16)
    got = codecs.dequant_q4_k(codes, _q4_k_plane(sc, m, d_bits, dmin_bits))
    for r in range(rows):
        for i in range(K):
            byte = int(codes[r, i // 2])
            q = (byte >> 4) if (i % 2) else (byte & 0xF)
            s = i // 256
            d = struct.unpack("<e", struct.pack("<H", int(d_bits[r, s])))[0]
            dmin = struct.unpack("<e", struct.pack("<H", int(dmin_bits[r, s])))[0]
            want = d * int(sc[r, i // 32]) * q - dmin * int(m[r, i // 32])
            assert got[r, i] == want, (r, i)


def test_q4_k_closed_forms():
    rows, K = 2, 256
    codes = np.arange(K // 2, dtype=np.uint8).reshape(1, -1).repeat(rows, 0)
    one = np.float16(1.0).view(np.uint16)
    zero = np.float16(0.0).view(np.uint16)
    full = lambda v: np.full((rows, K // 256), v, dtype=np.uint16)
    # d = 1, every scale 1, no min: the codes themselves
    w = codecs.dequant_q4_k(codes, _q4_k_plane(np.ones((rows, 8), int), np.zeros((rows, 8), int),
                                               full(one), full(zero)))
    q = np.empty((rows, K))
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    assert np.array_equal(w, q)
    # d = 0: only the min term, -dmin * m_b, constant over each block
    mins = np.arange(16).reshape(2, 8)
    w = codecs.dequant_q4_k(codes, _q4_k_plane(np.ones((rows, 8), int), mins, full(zero),
                                               full(one)))
    assert np.array_equal(w, -np.repeat(mins, 32, axis=1).astype(float))


def test_q5_k_brute_force_per_element():
    """Q5_K: each element's code rebuilt bit by bit (low nibble, then bit i of high byte j
    for element 8j + i) and its weight evaluated with Python floats."""
    import struct
    rng = np.random.default_rng(4)
    rows, K = 2, 512
    lo = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    hb = rng.integers(0, 256, size=(rows, K // 8), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(rows, K // 32))
    m = rng.integers(0, 64, size=(rows, K // 32))
    d_bits = rng.uniform(-1, 1, size=(rows, K // 256)).astype(np.float16).view(np.uint16)
    dmin_bits = rng.uniform(-1, 1, size=(rows, K // 256)).astype(np.float16).view(np.uint16)
    got = codecs.dequant_q5_k(np.concatenate([lo, hb], axis=1),
                              _q4_k_plane(sc, m, d_bits, dmin_bits))
    for r in range(rows):
        for i in range(K):
            byte = int(lo[r, i // 2])
            q = ((byte >> 4) if (i % 2) else (byte & 0xF)) + 16 * ((int(hb[r, i // 8]) >> (i % 8)) & 1)
            s = i // 256
            d = struct.unpack("<e", struct.pack("<H", int(d_bits[r, s])))[0]
            dmin = struct.unpack("<e", struct.pack("<H", int(dmin_bits[r, s])))[0]
            assert got[r, i] == d * int(sc[r, i // 32]) * q - dmin * int(m[r, i // 32]), (r, i)


def test_q5_k_reduces_to_q4_k_and_to_its_high_bits():
    rng = np.random.default_rng(5)
    rows, K = 2, 256
    lo = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(rows, K // 32))
    m = rng.integers(0, 64, size=(rows, K // 32))
    d_bits = rng.uniform(0, 1, size=(rows, 1)).astype(np.float16).view(np.uint16)
    dmin_bits = rng.uniform(0, 1, size=(rows, 1)).astype(np.float16).view(np.uint16)
    plane = _q4_k_plane(sc, m, d_bits, dmin_bits)
    # no high bits: the Q4_K matrix of the same low nibbles and scales
    zeros = np.zeros((rows, K // 8), dtype=np.uint8)
    assert np.array_equal(codecs.dequant_q5_k(np.concatenate([lo, zeros], axis=1), plane),
                          codecs.dequant_q4_k(lo, plane))
    # no low nibbles, every high bit set: 16 d sc - dmin m
    ones = np.full((rows, K // 8), 255, dtype=np.uint8)
    w = codecs.dequant_q5_k(np.concatenate([np.zeros_like(lo), ones], axis=1), plane)
    d = d_bits.view(np.float16).astype(np.float64)
    dmin = dmin_bits.view(np.float16).astype(np.float64)
    want = np.repeat(16 * d * sc - dmin * m, 32, axis=1)
    assert np.array_equal(w, want)


def _q6_k_plane(sc, d_bits):
    """Q6_K scale plane bytes written field by field with struct."""
    import struct
    rows, nsub = sc.shape
    out = np.zeros((rows, nsub + 2 * (nsub // 16)), dtype=np.uint8)
    for r in range(rows):
        raw = struct.pack(f"<{nsub}b", *[int(v) for v in sc[r]])
        raw += struct.pack(f"<{nsub // 16}H", *[int(v) for v in d_bits[r]])
        out[r] = np.frombuffer(raw, dtype=np.uint8)
    return out


def test_q6_k_brute_force_per_element():
    """Q6_K: each code rebuilt from its nibble and its 2-bit high part, each weight evaluated
    with Python floats and the fp16 d decoded by struct."""
    import struct
    rng = np.random.default_rng(6)
    rows, K = 2, 512
    lo = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    hi = rng.integers(0, 256, size=(rows, K // 4), dtype=np.uint8)
    sc = rng.integers(-128, 128, size=(rows, K // 16))
    d_bits = rng.uniform(-1, 1, size=(rows, K // 256)).astype(np.float16).view(np.uint16)
    got = codecs.dequant_q6_k(np.concatenate([lo, hi], axis=1), _q6_k_plane(sc, d_bits))
    for r in range(rows):
        for i in range(K):
            byte = int(lo[r, i // 2])
            q = ((byte >> 4) if (i % 2) else (byte & 0xF)) + 16 * ((int(hi[r, i // 4]) >> (2 * (i % 4))) & 3)
            d = struct.unpack("<e", struct.pack("<H", int(d_bits[r, i // 256])))[0]
            assert got[r, i] == d * int(sc[r, i // 16]) * (q - 32), (r, i)


def test_q6_k_closed_forms():
    rows, K = 1, 256
    one = np.full((rows, 1), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    # every code 32 (nibble 0, high part 2): all weights zero whatever the scales
    lo = np.zeros((rows, K // 2), dtype=np.uint8)
    hi = np.full((rows, K // 4), 0b10101010, dtype=np.uint8)
    sc = np.arange(-8, 8).reshape(1, 16) * 15
    w = codecs.dequant_q6_k(np.concatenate([lo, hi], axis=1), _q6_k_plane(sc, one))
    assert np.array_equal(w, np.zeros((rows, K)))
    # every code 63 with d = 1: 31 * sc of each 16-element sub-block
    lo = np.full((rows, K // 2), 0xFF, dtype=np.uint8)
    hi = np.full((rows, K // 4), 0xFF, dtype=np.uint8)
    w = codecs.dequant_q6_k(np.concatenate([lo, hi], axis=1), _q6_k_plane(sc, one))
    assert np.array_equal(w, np.repeat(31.0 * sc, 16, axis=1))
