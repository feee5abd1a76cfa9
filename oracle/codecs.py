"""Closed-form decoders for the number formats the routed MoE layer reads, in fp64.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py for who may use it).

The expert-offloading pages ask for the experts to be computed on their native
block-quantized bytes, with no bf16 copy of the weights (tinyserve README, opening
paragraph and "How it works" item 2; "What we tried and ruled out", last row).
They name the formats (MXFP4; GGUF Q8_0 in "Supported models" / "Formats") but do
not define them, so the definitions below are the public ones:
  * E2M1 (OCP Microscaling Formats v1.0): sign bit, 2 exponent bits (bias 1),
    1 mantissa bit, no inf/NaN; exponent 0 is subnormal (value m * 1/2).
  * E8M0 (same spec): an unsigned power-of-two scale 2^(b-127); b = 255 is NaN.
  * MXFP4 block: 32 E2M1 codes sharing one E8M0 scale.
  * Q8_0 block (GGUF): 32 two's-complement int8 codes sharing one fp16 scale d.
  * Q4_K (GGUF k-quant, named in "How it works" item 2 and "Formats"): super-blocks of
    256 elements made of eight 32-element blocks; block b has a 6-bit scale sc_b and a
    6-bit min m_b, the super-block an fp16 scale d and an fp16 min scale dmin; element
    value d*sc_b*q - dmin*m_b for its 4-bit code q (0..15). The byte arrangement of the
    scales is this library's own canonical one (see dequant_q4_k).
  * Q5_K (GGUF k-quant, same pages): Q4_K's scales and mins with a 5-bit code
    q = low nibble + 16 * high bit (0..31).
  * Q6_K (GGUF k-quant, same pages): super-blocks of 256 elements made of sixteen
    16-element sub-blocks, each with a signed 8-bit scale sc_j, and an fp16 scale d per
    super-block; a 6-bit code q = low nibble + 16 * (2-bit high part) (0..63); element
    value d * sc_j * (q - 32).
  * IEEE binary16 and bfloat16 (the upper 16 bits of an IEEE binary32).
Every function returns exact fp64 values; all of these formats embed exactly in fp64.
"""
from __future__ import annotations

import math
import numpy as np

# ---------------------------------------------------------------------------- scalars


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code, bits s e1 e0 m (s is the top bit)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return -mag if s else mag   # code 8 gives -0.0


def e8m0_value(b: int) -> float:
    """Value of an E8M0 scale byte: 2^(b - 127), NaN for 0xFF."""
    if b == 255:
        return math.nan
    return math.ldexp(1.0, b - 127)


def fp16_value(bits: int) -> float:
    """Value of an IEEE binary16 bit pattern."""
    s = (bits >> 15) & 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0:
        mag = math.ldexp(f, -24)                 # subnormal: f * 2^-14 * 2^-10
    elif e == 31:
        mag = math.inf if f == 0 else math.nan
    else:
        mag = math.ldexp(1024 + f, e - 25)       # (1 + f/1024) * 2^(e-15)
    return -mag if s else mag


def bf16_value(bits: int) -> float:
    """Value of a bfloat16 bit pattern: the binary32 whose upper half it is."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        mag = math.ldexp(f, -133)                # f * 2^-126 * 2^-7
    elif e == 255:
        mag = math.inf if f == 0 else math.nan
    else:
        mag = math.ldexp(128 + f, e - 134)       # (1 + f/128) * 2^(e-127)
    return -mag if s else mag


# ----------------------------------------------------------------------------- arrays

_E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return _E2M1_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    return _E8M0_TABLE[np.asarray(b, dtype=np.uint8)]


def fp16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (bits >> 15) & 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -24),
                   np.ldexp((1024 + f).astype(np.float64), (e - 25).astype(np.int64)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -133),
                   np.ldexp((128 + f).astype(np.float64), (e - 134).astype(np.int64)))
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even, in one step.

    Returns the rounded values as fp64 (exact). Normal range: 8 significant bits;
    below 2^-126 the spacing is fixed at 2^-133; values that round past the largest
    finite bf16 (just under 2^128) become +-inf.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    mag = np.abs(a)
    fin = np.isfinite(a)
    _, ex = np.frexp(mag)                    # mag = m * 2^ex, m in [0.5, 1)
    normal = fin & (mag >= 2.0 ** -126)
    # normal: keep 8 significant bits -> units of 2^(ex-8)
    q = np.rint(np.ldexp(mag, 8 - ex))       # exact scaling; rint is round-half-even
    r_norm = np.ldexp(q, ex - 8)
    sub = fin & ~normal
    r_sub = np.rint(np.ldexp(mag, 133)) * 2.0 ** -133
    r = np.where(normal, r_norm, np.where(sub, r_sub, mag))
    big = 2.0 ** 127 * (2.0 - 2.0 ** -7)     # largest finite bf16
    r = np.where(fin & (r > big), np.inf, r)
    out[...] = np.copysign(r, a)              # keeps the sign of -0
    out[np.isnan(a)] = np.nan
    return out


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """Bit patterns of fp64 values that are already exactly bf16 (e.g. bf16_round's output)."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


# ------------------------------------------------------------------ block dequantizers


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix [rows, K/2] codes + [rows, K/32] E8M0 scales -> fp64 [rows, K].

    Element 2j of a row is the low nibble of byte j, element 2j+1 the high nibble.
    Weight (r, i) = E2M1(code[r, i]) * 2^(scale[r, i // 32] - 127).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    K = 2 * half
    vals = np.empty((rows, K), dtype=np.float64)
    vals[:, 0::2] = e2m1_decode(codes & 0x0F)
    vals[:, 1::2] = e2m1_decode(codes >> 4)
    sc = e8m0_decode(scales)                        # [rows, K/32]
    return vals * np.repeat(sc, 32, axis=1)


def dequant_q8_0(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Q8_0 matrix [rows, K] int8 codes + [rows, K/32] fp16 scale bits -> fp64 [rows, K].

    Weight (r, i) = fp16(d[r, i // 32]) * q[r, i].
    """
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    sc = fp16_decode(d)
    return q * np.repeat(sc, 32, axis=1)


def q4_k_fields(scales: np.ndarray, K: int):
    """Split a Q4_K scale plane [rows, K/16 + K/64] (bytes) into its fields.

    Per row: K/32 pairs of bytes (sc_b, m_b), then K/256 pairs of little-endian fp16
    (d_s, dmin_s). Returns (sc, m) int [rows, K/32] and (d, dmin) fp64 [rows, K/256].
    """
    scales = np.asarray(scales, dtype=np.uint8)
    nb, ns = K // 32, K // 256
    pairs = scales[:, :2 * nb].reshape(-1, nb, 2).astype(np.int64)
    sup = np.ascontiguousarray(scales[:, 2 * nb:2 * nb + 4 * ns]).view(np.uint16)
    sup = sup.reshape(-1, ns, 2)
    return pairs[..., 0], pairs[..., 1], fp16_decode(sup[..., 0]), fp16_decode(sup[..., 1])


def dequant_q4_k(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q4_K matrix [rows, K/2] codes + [rows, K/16 + K/64] scale bytes -> fp64 [rows, K].

    Element 2j of a row is the low nibble of byte j, element 2j+1 the high nibble (as for
    MXFP4). Weight (r, i) = d[r, s] * sc[r, b] * q[r, i] - dmin[r, s] * m[r, b] with
    b = i // 32 and s = i // 256.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    K = 2 * half
    q = np.empty((rows, K), dtype=np.float64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    sc, m, d, dmin = q4_k_fields(scales, K)
    a = np.repeat(d, 8, axis=1) * sc                  # [rows, K/32]
    c = np.repeat(dmin, 8, axis=1) * m
    return q * np.repeat(a, 32, axis=1) - np.repeat(c, 32, axis=1)


def q5_k_codes(codes: np.ndarray) -> np.ndarray:
    """5-bit codes of a Q5_K code plane [rows, K/2 + K/8] -> int [rows, K].

    Per row: K/2 bytes of low nibbles (element 2j in the low nibble of byte j), then K/8
    bytes of high bits (element 8j + i in bit i of byte j).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, n = codes.shape
    K = n * 8 // 5
    lo = codes[:, :K // 2]
    hb = codes[:, K // 2:K // 2 + K // 8]
    q = np.empty((rows, K), dtype=np.int64)
    q[:, 0::2] = lo & 0x0F
    q[:, 1::2] = lo >> 4
    for i in range(8):
        q[:, i::8] += 16 * ((hb >> i) & 1)
    return q


def dequant_q5_k(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q5_K matrix [rows, K/2 + K/8] codes + [rows, K/16 + K/64] scale bytes (as Q4_K)
    -> fp64 [rows, K]: weight (r, i) = d[r, s] * sc[r, b] * q[r, i] - dmin[r, s] * m[r, b]."""
    q = q5_k_codes(codes).astype(np.float64)
    K = q.shape[1]
    sc, m, d, dmin = q4_k_fields(scales, K)
    a = np.repeat(d, 8, axis=1) * sc
    c = np.repeat(dmin, 8, axis=1) * m
    return q * np.repeat(a, 32, axis=1) - np.repeat(c, 32, axis=1)


def q6_k_codes(codes: np.ndarray) -> np.ndarray:
    """6-bit codes of a Q6_K code plane [rows, K/2 + K/4] -> int [rows, K].

    Per row: K/2 bytes of low nibbles (element 2j in the low nibble of byte j), then K/4
    bytes of 2-bit high parts (element 4j + i in bits 2i, 2i+1 of byte j).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, n = codes.shape
    K = n * 4 // 3
    lo = codes[:, :K // 2]
    hi = codes[:, K // 2:K // 2 + K // 4]
    q = np.empty((rows, K), dtype=np.int64)
    q[:, 0::2] = lo & 0x0F
    q[:, 1::2] = lo >> 4
    for i in range(4):
        q[:, i::4] += 16 * ((hi >> (2 * i)) & 3)
    return q


def dequant_q6_k(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q6_K matrix [rows, K/2 + K/4] codes + [rows, K/16 + K/128] scale bytes -> fp64.

    Scale plane per row: K/16 signed bytes sc_j (one per 16-element sub-block), then K/256
    little-endian fp16 d_s. Weight (r, i) = d[r, i // 256] * sc[r, i // 16] * (q[r, i] - 32).
    """
    q = q6_k_codes(codes).astype(np.float64)
    K = q.shape[1]
    scales = np.asarray(scales, dtype=np.uint8)
    sc = scales[:, :K // 16].view(np.int8).astype(np.float64)
    d = fp16_decode(np.ascontiguousarray(scales[:, K // 16:K // 16 + K // 128]).view(np.uint16))
    a = np.repeat(d, 16, axis=1) * sc                  # [rows, K/16]
    return (q - 32.0) * np.repeat(a, 16, axis=1)


def dequant(fmt: str, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    if fmt == "mxfp4":
        return dequant_mxfp4(codes, scales)
    if fmt == "q8_0":
        return dequant_q8_0(codes, scales)
    if fmt == "q4_k":
        return dequant_q4_k(codes, scales)
    if fmt == "q5_k":
        return dequant_q5_k(codes, scales)
    if fmt == "q6_k":
        return dequant_q6_k(codes, scales)
    raise ValueError(f"unknown block format {fmt!r}")
