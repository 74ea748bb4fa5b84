"""Q4_K simulated quantization (oracle; test infrastructure only).

Source: QATFactory project page, "Supported formats" table (Q4_K column:
unsigned INT4 elements, blocks of 32 inside a 256-element super-block, 6-bit
block scales under FP16 super-block scales, asymmetric, 4.50 bits per weight,
weight-only W4A16, served by llama.cpp).

Asymmetric means each 32-block carries a scale and a minimum (offset); 4.50
bits per weight for 256 weights is 256*4 + 8*(6+6) + 2*16 = 1152 bits = 144
bytes, which fixes the field sizes: 4-bit codes, a 6-bit scale and a 6-bit min
per sub-block, and two FP16 super-block values d (for scales) and dmin (for
mins).  The page does not give the quantizer; this oracle uses plain min/max
round-to-nearest (a stated choice), with the value model
    x_hat = d * sc_j * q - dmin * m_j,   q in 0..15, sc_j, m_j in 0..63.

Per super-block of 256 (row-major, along the contiguous axis), sub-block j:
1. mn_j = min(min x, 0); mx_j = max x.  (The min is clamped at or below 0 so
   the subtracted offset is non-negative.)  Comparisons are numeric (-0 equals
   +0) and a zero min or max is taken as +0, so no scale picks up a sign.
2. scale_j = fl(fl(mx_j - mn_j) / 15); off_j = fl(0 - mn_j).
3. d = fp16(fl(max_j scale_j / 63)); dmin = fp16(fl(max_j off_j / 63)).
4. sc_j = 0 if d == 0 else clamp(rint(fl(scale_j / d)), 0, 63);
   m_j = 0 if dmin == 0 else clamp(rint(fl(off_j / dmin)), 0, 63).
5. D_j = fl(d * sc_j), M_j = fl(dmin * m_j) (both exact).
6. q = 0 if D_j == 0 else clamp(rint(fl(fl(x + M_j) * fl(1 / D_j))), 0, 15).
7. Dequant: o = bf16(fl(D_j * q - M_j)) (D_j * q is exact: one rounding).

Packed super-block, 144 bytes (our own "GGUF-style" layout; llama.cpp's exact
bit arrangement is not available, so engine compatibility is parity unpinned):
bytes 0-1 d (fp16, little endian), 2-3 dmin, 4-15 a 96-bit little-endian bit
stream with sc_j at bits 6j..6j+5 and m_j at bits 48+6j..48+6j+5, bytes
16-143 the codes, byte i holding element 2i (low nibble) and 2i+1 (high).

A second sub-block scale rule, "mse", is kept as an option (a search of our own; the
page names an MSE-optimal quantizer only as a PTQ baseline and gives no rule): step 2's
scale_j is replaced by the best of 8 shrunken candidates, judged by the squared error of
the sub-block quantized with that scale and the offset off_j, before the two-level
(d, sc_j) quantization:
  base = fl(fl(mx_j - mn_j) / 15); for k = 0..7: s_k = fl(base * (1 - k/16));
  r = 0 if s_k == 0 else fl(1 / s_k); q_e = clamp(rint(fl(fl(x_e - mn_j) * r)), 0, 15);
  e_e = fl(fl(fl(q_e * s_k) + mn_j) - x_e); err_k = the sum of fl(e_e * e_e) in a fixed
  order: over the 8 elements of each quarter of the sub-block in index order, then
  (quarter 0 + quarter 1) + (quarter 2 + quarter 3), each addition rounded to float32;
  scale_j = s_k for the first k with the smallest err_k (k = 0 is the min/max rule).
Steps 3-7 are unchanged.

Pins: closed-form packed size, brute-force per-element q and rint steps,
on-grid outputs, QDQ == dequant(unpack(pack)), planted exact round trip and
idempotence, tests/test_oracle_formats.py; the mse rule in tests/test_oracle_q4k_mse.py.
"""

import numpy as np

from .primitives import (F32, bf16_to_f32, f32_to_bf16, f32_to_f16_bits, f16_bits_to_f32, rint)

SUPER = 256
SUB = 32
NSUB = SUPER // SUB
BLOCK_BYTES = 144


MSE_CANDIDATES = 8


def mse_scale(x, mn, mx):
    """Sub-block scales under the mse rule.  x: float32 [..., NSUB, SUB]; mn, mx: the
    sub-blocks' (normalized) extremes [..., NSUB].  Returns (scale [..., NSUB] float32,
    err [..., NSUB, MSE_CANDIDATES] float32, the chosen candidate index)."""
    base = ((mx - mn).astype(np.float32) / F32(15.0)).astype(np.float32)
    t = (x - mn[..., None]).astype(np.float32)                        # >= 0
    errs, scales = [], []
    for k in range(MSE_CANDIDATES):
        s = (base * F32(1.0 - k / 16.0)).astype(np.float32)
        zero = s == 0
        with np.errstate(divide="ignore"):
            r = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), s)).astype(np.float32)
        q = np.clip(rint((t * r[..., None]).astype(np.float32)), 0, 15).astype(np.float32)
        xh = ((q * s[..., None]).astype(np.float32) + mn[..., None]).astype(np.float32)
        e = (xh - x).astype(np.float32)
        sq = (e * e).astype(np.float32).reshape(e.shape[:-1] + (4, SUB // 4))
        part = sq[..., 0]
        for i in range(1, SUB // 4):                                    # in index order
            part = (part + sq[..., i]).astype(np.float32)
        err = ((part[..., 0] + part[..., 1]).astype(np.float32) +
               (part[..., 2] + part[..., 3]).astype(np.float32)).astype(np.float32)
        errs.append(err)
        scales.append(s)
    err = np.stack(errs, axis=-1)
    best = np.zeros(err.shape[:-1], np.int64)
    best_err = err[..., 0]
    for k in range(1, MSE_CANDIDATES):                                 # first strict minimum
        better = err[..., k] < best_err
        best = np.where(better, k, best)
        best_err = np.where(better, err[..., k], best_err)
    scale = np.take_along_axis(np.stack(scales, axis=-1), best[..., None], axis=-1)[..., 0]
    return scale.astype(np.float32), err, best


def quantize(x_bits, rule="minmax"):
    """Returns dict with d, dmin (fp16 bits [rows, nsb]), sc, m ([rows, nsb, 8] uint8),
    q ([rows, cols] uint8).  rule: "minmax" (the default) or "mse" (see the module notes)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    assert cols % SUPER == 0
    nsb = cols // SUPER
    x = bf16_to_f32(x_bits).reshape(rows, nsb, NSUB, SUB)
    if cols == 0:
        z = np.zeros((rows, 0), np.uint16)
        return dict(d=z, dmin=z, sc=np.zeros((rows, 0, NSUB), np.uint8),
                    m=np.zeros((rows, 0, NSUB), np.uint8), q=np.zeros((rows, 0), np.uint8))
    # min and max compare numerically (-0 == +0); a zero result is taken as +0
    mn = np.minimum(np.min(x, axis=-1), F32(0.0))
    mn = np.where(mn == 0, F32(0.0), mn).astype(np.float32)
    mx = np.max(x, axis=-1)
    mx = np.where(mx == 0, F32(0.0), mx).astype(np.float32)
    if rule == "minmax":
        scale = ((mx - mn).astype(np.float32) / F32(15.0)).astype(np.float32)
    elif rule == "mse":
        scale = mse_scale(x, mn, mx)[0]
    else:
        raise ValueError(rule)
    off = (F32(0.0) - mn).astype(np.float32)
    d_bits = f32_to_f16_bits((np.max(scale, axis=-1) / F32(63.0)).astype(np.float32))
    dmin_bits = f32_to_f16_bits((np.max(off, axis=-1) / F32(63.0)).astype(np.float32))
    d = f16_bits_to_f32(d_bits)[..., None]
    dmin = f16_bits_to_f32(dmin_bits)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d == 0, 0.0, np.clip(rint((scale / np.where(d == 0, F32(1), d)).astype(np.float32)), 0, 63))
        m = np.where(dmin == 0, 0.0, np.clip(rint((off / np.where(dmin == 0, F32(1), dmin)).astype(np.float32)), 0, 63))
    sc = sc.astype(np.uint8)
    m = m.astype(np.uint8)
    D = (d * sc.astype(np.float32)).astype(np.float32)
    M = (dmin * m.astype(np.float32)).astype(np.float32)
    Dz = D == 0
    r = (F32(1.0) / np.where(Dz, F32(1.0), D)).astype(np.float32)
    t = ((x + M[..., None]).astype(np.float32) * r[..., None]).astype(np.float32)
    q = np.clip(rint(t), 0, 15)
    q = np.where(Dz[..., None], 0, q).astype(np.uint8)
    return dict(d=d_bits, dmin=dmin_bits, sc=sc, m=m, q=q.reshape(rows, cols))


def dequantize(p):
    """BF16 bits of bf16(fl(D_j * q - M_j))."""
    q = p["q"]
    rows, cols = q.shape
    nsb = cols // SUPER
    d = f16_bits_to_f32(p["d"])[..., None]
    dmin = f16_bits_to_f32(p["dmin"])[..., None]
    D = (d * p["sc"].astype(np.float32)).astype(np.float32)[..., None]
    M = (dmin * p["m"].astype(np.float32)).astype(np.float32)[..., None]
    qq = q.reshape(rows, nsb, NSUB, SUB).astype(np.float32)
    o = ((D * qq).astype(np.float32) - M).astype(np.float32)
    return f32_to_bf16(o).reshape(rows, cols).astype(np.uint16)


def qdq(x_bits, rule="minmax"):
    return dequantize(quantize(x_bits, rule))


def pack(p):
    """[rows, nsb, 144] uint8 blocks."""
    q = p["q"]
    rows, cols = q.shape
    nsb = cols // SUPER
    out = np.zeros((rows, nsb, BLOCK_BYTES), dtype=np.uint8)
    d = np.asarray(p["d"], np.uint16)
    dmin = np.asarray(p["dmin"], np.uint16)
    out[..., 0] = d & 0xFF
    out[..., 1] = d >> 8
    out[..., 2] = dmin & 0xFF
    out[..., 3] = dmin >> 8
    # 96-bit stream as a Python-int-free pair of 48-bit halves
    sc = p["sc"].astype(np.uint64)
    m = p["m"].astype(np.uint64)
    lo = np.zeros((rows, nsb), np.uint64)
    hi = np.zeros((rows, nsb), np.uint64)
    for j in range(NSUB):
        lo |= sc[..., j] << np.uint64(6 * j)
        hi |= m[..., j] << np.uint64(6 * j)
    for byte in range(6):
        out[..., 4 + byte] = ((lo >> np.uint64(8 * byte)) & np.uint64(0xFF)).astype(np.uint8)
        out[..., 10 + byte] = ((hi >> np.uint64(8 * byte)) & np.uint64(0xFF)).astype(np.uint8)
    qq = q.reshape(rows, nsb, SUPER)
    out[..., 16:] = (qq[..., 0::2] | (qq[..., 1::2] << 4)).astype(np.uint8)
    return out


def unpack(blocks):
    blocks = np.asarray(blocks, dtype=np.uint8)
    rows, nsb, _ = blocks.shape
    d = (blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8))
    dmin = (blocks[..., 2].astype(np.uint16) | (blocks[..., 3].astype(np.uint16) << 8))
    lo = np.zeros((rows, nsb), np.uint64)
    hi = np.zeros((rows, nsb), np.uint64)
    for byte in range(6):
        lo |= blocks[..., 4 + byte].astype(np.uint64) << np.uint64(8 * byte)
        hi |= blocks[..., 10 + byte].astype(np.uint64) << np.uint64(8 * byte)
    sc = np.stack([(lo >> np.uint64(6 * j)) & np.uint64(63) for j in range(NSUB)], axis=-1).astype(np.uint8)
    m = np.stack([(hi >> np.uint64(6 * j)) & np.uint64(63) for j in range(NSUB)], axis=-1).astype(np.uint8)
    q = np.empty((rows, nsb, SUPER), np.uint8)
    q[..., 0::2] = blocks[..., 16:] & 0x0F
    q[..., 1::2] = blocks[..., 16:] >> 4
    return dict(d=d.astype(np.uint16), dmin=dmin.astype(np.uint16), sc=sc, m=m, q=q.reshape(rows, nsb * SUPER))


def packed_bytes(rows, cols):
    return rows * (cols // SUPER) * BLOCK_BYTES
