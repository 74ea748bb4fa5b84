"""NVFP4 simulated quantization (oracle; test infrastructure only).

Source: QATFactory project page, "Supported formats" table (NVFP4 column:
E2M1 elements, block size 16, block E4M3 scale plus tensor FP32 scale,
symmetric, 4.50 bits per weight) and "Method" section, "Deployment-aligned
simulated quantization" (projections the engines fuse, such as QKV and gate/up,
share one tensor scale).

Readings of what the page leaves open (each a stated choice):

* Blocks are 16 consecutive elements along the contiguous (input / K) axis of
  a row-major [rows, cols] tensor.
* Tensor scale of a tied group g: A = max |x| over every element of every
  tensor in g (exact); s_t = 1 if A == 0, else fl(A / 2688).  2688 = 6 * 448 =
  largest E2M1 magnitude times largest E4M3 value, so the group's largest
  block lands at the top of the E4M3 range.
* Block scale: k = fl(6 * s_t); a = max |x| over the block; u = fl(a / k);
  S = E4M3 RNE-satfinite(u); s = value(S).
* Element code: d = fl(s * s_t).  If d == 0 every magnitude code is 0.
  Otherwise r = fl(1 / d) (one correctly rounded reciprocal per block),
  y = fl(|x| * r), magnitude = E2M1 RNE-saturating(y).  The code's sign bit is
  x's sign bit, also for -0.0 and for negatives that round to magnitude 0.
* Dequant: o = sign * bf16(fl(fl(v * s) * s_t)), v the E2M1 magnitude
  (v * s is exact, so there are exactly two roundings: fp32 then bf16).

Packing (a "compressed-tensors-style" layout of our own; byte-level engine
compatibility is parity unpinned because no engine spec is available):
codes[r][c/2] holds element 2i in the low nibble and 2i+1 in the high nibble;
scales[r][c/16] holds E4M3 bytes; the fp32 tensor scale s_t travels separately
(per tied group).  9 bytes per 16 elements plus 4 bytes per group, i.e. 4.50
bits per weight, as the table states.

Tracked scale (activations): the running maximum of |x| over the batches seen so far,
then the rule above; see tracked_scale.

Pins: closed-form packed size (bits per weight from the table), brute-force
element codes, on-grid outputs, QDQ == dequant(unpack(pack)), idempotence for
normal block scales, exact-representable round trip, tying equals fusing,
tests/test_oracle_formats.py; the tracked scale equals the scale of all batches
seen so far taken together, in any order, tests/test_oracle_misc.py.
"""

import numpy as np

from .primitives import (F32, bf16_to_f32, f32_to_bf16, e2m1_encode_mag, E2M1_MAG,
                         e4m3_encode, e4m3_value)

BLOCK = 16
TENSOR_DIV = F32(2688.0)        # 6 * 448


def group_amax(tensors):
    """A = max |x| over all elements of the tensors of one tied group (float32).

    Returns (A, nonfinite) where nonfinite is True when any element is Inf/NaN.
    """
    A = F32(0.0)
    nonfinite = False
    for t in tensors:
        v = bf16_to_f32(t)
        if v.size == 0:
            continue
        if not np.all(np.isfinite(v)):
            nonfinite = True
        m = np.max(np.abs(v))
        if m > A or np.isnan(m):
            A = F32(m)
    return A, nonfinite


def tensor_scale(tensors):
    """FP32 tensor scale s_t shared by one tied group: 1 if A == 0 else fl(A / 2688)."""
    A, _ = group_amax(tensors)
    if A == 0:
        return F32(1.0)
    return F32(A) / TENSOR_DIV


def tracked_scale(amax_prev, tensors):
    """Tracked tensor scale ("Method", "Export" on the project page: NVFP4 activation
    scales are tracked during training and saved, so no calibration pass runs).  Reading:
    the tracked amax is the running maximum of |x| over every batch seen so far.
    Returns (amax, s_t): amax = max(amax_prev, A of this batch's tied group) as float32,
    s_t = 1 if amax == 0 else fl(amax / 2688) (the rule of tensor_scale)."""
    A, _ = group_amax(tensors)
    amax = max(F32(amax_prev), F32(A))
    return F32(amax), (F32(1.0) if amax == 0 else F32(amax) / TENSOR_DIV)


def _scaled(x_bits, s_t):
    """The quantizer's intermediate values for x [rows, cols]: (x as float32 blocks
    [rows, cols/16, 16], y = fl(|x| r) per element, the E4M3 codes S, d == 0 per block)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    assert cols % BLOCK == 0
    s_t = F32(s_t)
    x = bf16_to_f32(x_bits).reshape(rows, cols // BLOCK, BLOCK)
    ax = np.abs(x)
    a = np.max(ax, axis=-1) if cols else np.zeros((rows, 0), np.float32)
    k = F32(6.0) * s_t
    u = (a / k).astype(np.float32)
    S = e4m3_encode(u)
    s = e4m3_value(S)
    d = (s * s_t).astype(np.float32)
    zero = d == 0
    with np.errstate(divide="ignore", over="ignore"):
        r = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), d)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (ax * r[..., None]).astype(np.float32)
    return x, y, S, zero


def quantize(x_bits, s_t):
    """Codes (uint8 per element, 0..15) and E4M3 block-scale codes for x [rows, cols]."""
    rows, cols = np.shape(x_bits)
    x, y, S, zero = _scaled(x_bits, s_t)
    mag = e2m1_encode_mag(y)
    mag[np.broadcast_to(zero[..., None], mag.shape)] = 0
    sign = np.signbit(x).astype(np.uint8)
    codes = (sign << 3) | mag
    return codes.reshape(rows, cols), S


def saturated(x_bits, s_t):
    """Elements the quantizer saturates: the scaled magnitude y = fl(|x| r) exceeds 6, the
    largest E2M1 magnitude (bool [rows, cols]).  Blocks with d == 0 have none; a zero
    element has none even where r overflowed (0 * inf is no magnitude)."""
    rows, cols = np.shape(x_bits)
    x, y, S, zero = _scaled(x_bits, s_t)
    with np.errstate(invalid="ignore"):
        sat = (y > F32(6.0)) & ~zero[..., None] & (x != 0)
    return sat.reshape(rows, cols)


def dequantize(codes, S, s_t):
    """BF16 bits of the dequantized values: sign | bf16(fl(fl(v * s) * s_t))."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    c = codes.reshape(rows, cols // BLOCK, BLOCK)
    v = E2M1_MAG[c & 7].astype(np.float32)
    s = e4m3_value(S)[..., None]
    o = ((v * s).astype(np.float32) * F32(s_t)).astype(np.float32)
    bits = f32_to_bf16(o) | ((c >> 3).astype(np.uint16) << np.uint16(15))
    return bits.reshape(rows, cols).astype(np.uint16)


def qdq(x_bits, s_t):
    """BF16 bits of QDQ(x) under one tensor scale."""
    codes, S = quantize(x_bits, s_t)
    return dequantize(codes, S, s_t)


def pack(codes, S):
    """(packed codes [rows, cols/2] uint8, scales [rows, cols/16] uint8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[:, 0::2]
    hi = codes[:, 1::2]
    return (lo | (hi << 4)).astype(np.uint8), np.asarray(S, dtype=np.uint8).copy()


def unpack(packed, scales):
    """Inverse of pack: (codes [rows, cols], S [rows, cols/16])."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, half * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes, np.asarray(scales, dtype=np.uint8)


def packed_bytes(rows, cols, n_groups=1):
    """Bytes of the packed form: cols/2 code bytes + cols/16 scale bytes per row, 4 per group."""
    return rows * (cols // 2) + rows * (cols // BLOCK) + 4 * n_groups
