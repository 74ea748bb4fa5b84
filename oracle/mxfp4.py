"""MXFP4 simulated quantization (oracle; test infrastructure only).

Source: QATFactory project page, "Supported formats" table (MXFP4 column:
E2M1 elements, block size 32, block E8M0 scale, symmetric, 4.25 bits per
weight; no tensor-level scale, hence no tying, per the "Deployment-aligned
simulated quantization" paragraph of the "Method" section).

Readings of what the page leaves open (stated choices):

* Blocks are 32 consecutive elements along the contiguous axis.
* Shared exponent: a = max |x| over the block.  a == 0 gives E = 0.
  Otherwise e = floor(log2 a) (exact from the bf16 bits) and
  E = clamp(e - 2 + 127, 0, 254): the exponent of the largest element minus
  the largest E2M1 exponent (2), the usual microscaling rule.  Blocks whose
  amax lies in (6, 8) * 2^(E-127) therefore clip their top element to 6.
* A second shared-exponent rule, "noclip", is kept as an option (the pages do not fix
  the rule): E = the smallest value in [0, 252] with a <= 6 * 2^(E-127), i.e.
  ceil(log2(a / 6)) + 127 clamped to [0, 252], so that no element is clipped unless
  a > 6 * 2^125.  The upper end 252 is the largest exponent whose grid top 6 * 2^(E-127)
  is a finite bf16: at E = 253 a block maximum in [1.75, 2) * 2^127 would round to the
  code 4 and dequantize to 2^128, which bf16 cannot hold.  So blocks with maxima above
  1.5 * 2^127 take E = 252 and clip to 6 * 2^125, as under the floor rule (which never
  goes above 252 for finite inputs).
* X = 2^(E-127); y = |x| / X (exact unless it underflows far below 0.25);
  magnitude = E2M1 RNE-saturating(y); the code's sign bit is x's sign bit.
* Dequant: o = sign * bf16(v * X), exact, including bf16 subnormals.

Packing: codes[r][c/2] (element 2i low nibble, 2i+1 high nibble) and
scales[r][c/32] E8M0 bytes: 17 bytes per 32 elements = 4.25 bits per weight.
Engine compatibility is parity unpinned.

Pins: closed-form packed size, brute-force codes and exponents, on-grid outputs,
finite outputs for every finite input under both rules, QDQ == dequant(unpack(pack)),
exact idempotence on all finite inputs, exact-representable round trip;
tests/test_oracle_formats.py.
"""

import numpy as np

from .primitives import (F32, bf16_to_f32, f32_to_bf16, e2m1_encode_mag, E2M1_MAG,
                         e8m0_value, floor_log2)

BLOCK = 32
# the largest shared exponent of the noclip rule: 6 * 2^(252-127) = 1.5 * 2^127 is the
# top of the E2M1 grid that bf16 still holds; 6 * 2^126 is beyond the bf16 range
NOCLIP_E_MAX = 252


def shared_exponent(a, rule="floor"):
    """E8M0 byte of blocks with maxima a (float32 >= 0) under the floor or noclip rule."""
    a = np.asarray(a, dtype=np.float32)
    pos = a > 0
    e = np.where(pos, floor_log2(np.where(pos, a, 1.0)), 0)
    if rule == "floor":
        E = np.clip(e - 2 + 127, 0, 254)
    elif rule == "noclip":
        # the smallest E with a <= 6 * 2^(E - 127): a lies in [2^e, 2^(e+1)), so 6 * 2^(E-127)
        # first reaches it at E - 127 = e - 2 or e - 1; test both exactly in float64
        lo = e - 2 + 127
        fits = a.astype(np.float64) <= np.ldexp(6.0, lo - 127)
        E = np.clip(np.where(fits, lo, lo + 1), 0, NOCLIP_E_MAX)
    else:
        raise ValueError(rule)
    return np.where(pos, E, 0).astype(np.int64)


def quantize(x_bits, rule="floor"):
    """Codes (uint8 per element) and E8M0 scale bytes [rows, cols/32] for x [rows, cols]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    assert cols % BLOCK == 0
    x = bf16_to_f32(x_bits).reshape(rows, cols // BLOCK, BLOCK)
    ax = np.abs(x)
    a = np.max(ax, axis=-1) if cols else np.zeros((rows, 0), np.float32)
    E = shared_exponent(a, rule)
    X = e8m0_value(E)
    with np.errstate(under="ignore"):
        y = (ax / X[..., None]).astype(np.float32)
    mag = e2m1_encode_mag(y)
    sign = np.signbit(x).astype(np.uint8)
    codes = (sign << 3) | mag
    return codes.reshape(rows, cols), E.astype(np.uint8)


def saturated(x_bits, rule="floor"):
    """Elements the quantizer saturates: y = |x| / 2^(E-127) (exact) exceeds 6, the largest
    E2M1 magnitude (bool [rows, cols]).  Under the floor rule these are the elements in
    (6, 8) * 2^(E-127) of blocks whose maximum has a significand above 1.5; under the
    noclip rule only the elements above 6 * 2^125 = 1.5 * 2^127 (blocks capped at E = 252)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    x = bf16_to_f32(x_bits).reshape(rows, cols // BLOCK, BLOCK)
    ax = np.abs(x)
    a = np.max(ax, axis=-1) if cols else np.zeros((rows, 0), np.float32)
    X = e8m0_value(shared_exponent(a, rule))
    with np.errstate(under="ignore"):
        y = (ax / X[..., None]).astype(np.float32)
    return (y > F32(6.0)).reshape(rows, cols)


def dequantize(codes, E):
    """BF16 bits of sign * bf16(v * 2^(E-127))."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    c = codes.reshape(rows, cols // BLOCK, BLOCK)
    v = E2M1_MAG[c & 7].astype(np.float32)
    X = e8m0_value(np.asarray(E, dtype=np.int64))[..., None]
    o = (v * X).astype(np.float32)
    bits = f32_to_bf16(o) | ((c >> 3).astype(np.uint16) << np.uint16(15))
    return bits.reshape(rows, cols).astype(np.uint16)


def qdq(x_bits, rule="floor"):
    codes, E = quantize(x_bits, rule)
    return dequantize(codes, E)


def pack(codes, E):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), np.asarray(E, np.uint8).copy()


def unpack(packed, scales):
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, half * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes, np.asarray(scales, dtype=np.uint8)


def packed_bytes(rows, cols):
    return rows * (cols // 2) + rows * (cols // BLOCK)
