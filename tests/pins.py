"""Independent checks ("pins") of the oracle's format functions.

Every check recomputes what it needs by a route other than the oracle's own
code: float64 arithmetic rounded once to float32 (exact for a single +, -, *
or / of float32 operands, since 53 >= 2*24 + 2), Python's ``math.frexp`` and
``struct`` half-float packing, torch's casts, and brute-force searches over
every code.  Each returns the number of violations (0 = pass) so that the
mutation tests can show that a planted mistake in the oracle is caught.
"""

import math
import struct

import numpy as np
import torch

from oracle import primitives as P
from oracle import nvfp4, mxfp4, q4k

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def f32(x):
    """Round a float64 value (or array) to float32: one RNE rounding."""
    return np.asarray(x, np.float64).astype(np.float32)


def bf16_torch(x):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_torch(u):
    t = torch.from_numpy(np.minimum(np.asarray(u, np.float32), np.float32(448.0)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_val_torch(code):
    return torch.from_numpy(np.asarray(code, np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def f16_struct(x):
    """fp16 bits through Python's own binary16 packing (RNE), saturating at 65504."""
    out = np.empty(np.shape(x), np.uint16)
    for i, v in np.ndenumerate(np.asarray(x, np.float64)):
        v = max(-65504.0, min(65504.0, float(v)))
        out[i] = struct.unpack("<H", struct.pack("<e", v))[0]
    return out


def f16_val(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def best_codes(y, ties_even=True):
    """Set of acceptable E2M1 magnitude codes per value y (exact argmin; ties -> even)."""
    y = np.minimum(np.asarray(y, np.float64), 2.0 ** 40)
    dist = np.abs(y[..., None] - E2M1)
    ismin = dist == dist.min(axis=-1, keepdims=True)
    idx = np.arange(8)
    tie = ismin.sum(axis=-1) > 1
    even = np.where(ismin & (idx % 2 == 0), idx, 99).min(axis=-1)
    first = np.where(ismin, idx, 99).min(axis=-1)
    out = np.where(tie, even, first)
    return np.where(np.isnan(y), 0, out)


# --------------------------------------------------------------- NVFP4 -----
def nvfp4_scale_chain(x_bits, s_t):
    """Block scale codes, d and r per 16-block recomputed in float64 -> float32."""
    rows, cols = x_bits.shape
    x = widen(x_bits).reshape(rows, cols // 16, 16)
    a = np.abs(x).max(axis=-1)
    k = f32(6.0 * float(s_t))
    u = f32(a / np.float64(k))
    S = e4m3_torch(u)
    s = e4m3_val_torch(S)
    d = f32(s * float(s_t))
    with np.errstate(divide="ignore"):
        r = np.where(d == 0, 0.0, f32(1.0 / np.where(d == 0, 1.0, d.astype(np.float64))))
    return x, S, d.astype(np.float64), r.astype(np.float64)


def check_nvfp4(x_bits, s_t):
    """Violations of: scales, brute-force codes, signs, dequant values, pack round trip."""
    codes, S = nvfp4.quantize(x_bits, s_t)
    x, S_ref, d, r = nvfp4_scale_chain(x_bits, s_t)
    bad = int(np.sum(S != S_ref))
    rows, cols = x_bits.shape
    c = codes.reshape(rows, cols // 16, 16)
    with np.errstate(invalid="ignore", over="ignore"):
        y = f32(np.abs(x) * r[..., None]).astype(np.float64)
    want = np.where((d == 0)[..., None], 0, best_codes(y))
    bad += int(np.sum((c & 7) != want))
    bad += int(np.sum((c >> 3) != np.signbit(x)))
    # dequant: sign | bf16(fl(fl(v*s)*s_t)), each fl recomputed via float64
    s = e4m3_val_torch(S)[..., None]
    o = f32(f32(E2M1[c & 7] * s).astype(np.float64) * float(s_t))
    ref = (bf16_torch(o) | ((c >> 3).astype(np.uint16) << 15)).reshape(rows, cols)
    out = nvfp4.dequantize(codes, S, s_t)
    bad += int(np.sum(out != ref))
    pc, ps = nvfp4.pack(codes, S)
    bad += int(pc.size + ps.size != rows * cols // 2 + rows * cols // 16)
    # nibble order: element 2i low, 2i+1 high
    bad += int(np.sum((pc & 15) != codes[:, 0::2])) + int(np.sum((pc >> 4) != codes[:, 1::2]))
    u_codes, u_S = nvfp4.unpack(pc, ps)
    bad += int(np.sum(nvfp4.dequantize(u_codes, u_S, s_t) != nvfp4.qdq(x_bits, s_t)))
    return bad


def check_nvfp4_dequant(codes, S, s_t):
    """Violations of dequant(codes, S, s_t) == sign | bf16(fl(fl(v * s) * s_t))."""
    rows, cols = codes.shape
    c = codes.reshape(rows, cols // 16, 16)
    s = e4m3_val_torch(S)[..., None]
    o = f32(f32(E2M1[c & 7] * s).astype(np.float64) * float(s_t))
    ref = (bf16_torch(o) | ((c >> 3).astype(np.uint16) << 15)).reshape(rows, cols)
    return int(np.sum(nvfp4.dequantize(codes, S, s_t) != ref))


def check_nvfp4_tensor_scale(tensors):
    A = max(float(np.abs(widen(t)).max()) if t.size else 0.0 for t in tensors)
    want = np.float32(1.0) if A == 0 else f32(A / 2688.0)
    got = nvfp4.tensor_scale(tensors)
    return int(np.float32(got).view(np.uint32) != np.float32(want).view(np.uint32))


# --------------------------------------------------------------- MXFP4 -----
def check_mxfp4(x_bits):
    codes, E = mxfp4.quantize(x_bits)
    rows, cols = x_bits.shape
    x = widen(x_bits).reshape(rows, cols // 32, 32)
    a = np.abs(x).max(axis=-1)
    E_ref = np.zeros(a.shape, np.int64)
    for idx, ai in np.ndenumerate(a):
        if ai > 0:
            _, ex = math.frexp(ai)                 # ai = m * 2^ex, m in [0.5, 1)
            E_ref[idx] = min(max(ex - 1 - 2 + 127, 0), 254)
    bad = int(np.sum(E.astype(np.int64) != E_ref))
    X = np.ldexp(1.0, E_ref - 127)[..., None]
    y = np.abs(x) / X                              # exact in float64
    c = codes.reshape(rows, cols // 32, 32)
    bad += int(np.sum((c & 7) != best_codes(f32(y))))
    bad += int(np.sum((c >> 3) != np.signbit(x)))
    ref = (bf16_torch(f32(E2M1[c & 7] * X)) | ((c >> 3).astype(np.uint16) << 15)).reshape(rows, cols)
    bad += int(np.sum(mxfp4.dequantize(codes, E) != ref))
    pc, ps = mxfp4.pack(codes, E)
    bad += int(np.sum((pc & 15) != codes[:, 0::2])) + int(np.sum((pc >> 4) != codes[:, 1::2]))
    bad += int(np.sum(mxfp4.dequantize(*mxfp4.unpack(pc, ps)) != mxfp4.qdq(x_bits)))
    return bad


def planted_mx_blocks():
    """Block maxima on both sides of every decision of the noclip rule: 6 * 2^k exactly,
    one bf16 step above and below, mantissas 1.5 and 1.5 + one step, the smallest and
    largest normals, subnormals, zero."""
    vals = []
    for k in (-130, -126, -100, -3, 0, 1, 5, 100, 125):
        base = np.float32(np.ldexp(6.0, k))
        b = P.f32_to_bf16(np.array([base], np.float32))[0]
        vals += [int(b), int(b) + 1, int(b) - 1]
    for e in (1, 2, 3, 127, 254):
        vals += [(e << 7) | 0x40, (e << 7) | 0x41, (e << 7) | 0x3F, (e << 7) | 0x7F, e << 7]
    vals += [0x0001, 0x007F, 0x0000, 0x7F7F]
    vals = [v for v in vals if 0 <= v < 0x7F80]
    blocks = np.zeros((len(vals), 32), np.uint16)
    rng = np.random.default_rng(5)
    for i, v in enumerate(vals):
        lo = P.bf16_to_f32(np.array([v], np.uint16))[0]
        filler = P.f32_to_bf16((rng.uniform(-1, 1, 31) * lo).astype(np.float32))
        blocks[i, :31] = filler
        blocks[i, 31] = v | (0x8000 if i % 2 else 0)          # the block maximum, either sign
    return blocks


# the largest finite bf16, (2 - 2^-7) * 2^127, read from its bit pattern
BF16_MAX = struct.unpack("<f", struct.pack("<I", 0x7F7F0000))[0]


def noclip_exponents():
    """E8M0 bytes the noclip rule may use: those whose whole E2M1 grid, up to 6 * 2^(E-127),
    is a finite bf16 (so a QDQ'd value can never become Inf)."""
    return [k for k in range(255) if math.ldexp(6.0, k - 127) <= BF16_MAX]


def check_mxfp4_noclip(x_bits):
    """The noclip shared exponent by brute force over the usable E8M0 bytes: the smallest E
    with max|x| <= 6 * 2^(E-127) (exact in float64), or the largest usable one when none
    fits; then the same element rule as above."""
    codes, E = mxfp4.quantize(x_bits, rule="noclip")
    rows, cols = x_bits.shape
    x = widen(x_bits).reshape(rows, cols // 32, 32)
    a = np.abs(x).max(axis=-1)
    usable = noclip_exponents()
    E_ref = np.zeros(a.shape, np.int64)
    for idx, ai in np.ndenumerate(a):
        if ai > 0:
            E_ref[idx] = next((k for k in usable if ai <= math.ldexp(6.0, k - 127)), usable[-1])
    bad = int(np.sum(E.astype(np.int64) != E_ref))
    X = np.ldexp(1.0, E_ref - 127)[..., None]
    y = np.abs(x) / X
    c = codes.reshape(rows, cols // 32, 32)
    bad += int(np.sum((c & 7) != best_codes(f32(y))))
    bad += int(np.sum((c >> 3) != np.signbit(x)))
    return bad


# ---------------------------------------------------------------- Q4_K -----
def check_q4k(x_bits):
    p = q4k.quantize(x_bits)
    rows, cols = x_bits.shape
    nsb = cols // 256
    x = widen(x_bits).reshape(rows, nsb, 8, 32)
    mn = np.minimum(x.min(axis=-1), 0.0) + 0.0       # -0 + 0 = +0: zero extremes are +0
    mx = x.max(axis=-1) + 0.0
    scale = f32(f32(mx - mn).astype(np.float64) / 15.0).astype(np.float64)
    off = 0.0 - mn
    d_ref = f16_struct(f32(scale.max(axis=-1) / 63.0))
    dmin_ref = f16_struct(f32(off.max(axis=-1) / 63.0))
    bad = int(np.sum(p["d"] != d_ref)) + int(np.sum(p["dmin"] != dmin_ref))
    d = f16_val(d_ref)[..., None]
    dmin = f16_val(dmin_ref)[..., None]
    # sc_j, m_j: brute force over 0..63 of |t - k| with t = fl(scale / d), ties to even k
    ks = np.arange(64)

    def argmin_int(t, valid):
        dist = np.abs(t[..., None] - ks)
        ismin = dist == dist.min(axis=-1, keepdims=True)
        tie = ismin.sum(axis=-1) > 1
        even = np.where(ismin & (ks % 2 == 0), ks, 999).min(axis=-1)
        first = np.where(ismin, ks, 999).min(axis=-1)
        return np.where(valid, np.where(tie, even, first), 0)

    with np.errstate(divide="ignore", invalid="ignore"):
        t_sc = f32(scale / np.where(d == 0, 1.0, d)).astype(np.float64)
        t_m = f32(off / np.where(dmin == 0, 1.0, dmin)).astype(np.float64)
    sc_ref = argmin_int(t_sc, np.broadcast_to(d != 0, t_sc.shape))
    m_ref = argmin_int(t_m, np.broadcast_to(dmin != 0, t_m.shape))
    bad += int(np.sum(p["sc"] != sc_ref)) + int(np.sum(p["m"] != m_ref))
    D = d * sc_ref
    M = dmin * m_ref                                # exact products
    with np.errstate(divide="ignore"):
        r = np.where(D == 0, 0.0, f32(1.0 / np.where(D == 0, 1.0, D)).astype(np.float64))
    t = f32(f32(x + M[..., None]).astype(np.float64) * r[..., None]).astype(np.float64)
    qs = np.arange(16)
    dist = np.abs(t[..., None] - qs)
    ismin = dist == dist.min(axis=-1, keepdims=True)
    tie = ismin.sum(axis=-1) > 1
    even = np.where(ismin & (qs % 2 == 0), qs, 99).min(axis=-1)
    first = np.where(ismin, qs, 99).min(axis=-1)
    q_ref = np.where((D == 0)[..., None], 0, np.where(tie, even, first))
    bad += int(np.sum(p["q"].reshape(q_ref.shape) != q_ref))
    o = f32(D[..., None] * q_ref - M[..., None])      # D*q exact; one rounding
    bad += int(np.sum(q4k.dequantize(p) != bf16_torch(o).reshape(rows, cols)))
    blocks = q4k.pack(p)
    bad += int(blocks.size != rows * nsb * 144)
    u = q4k.unpack(blocks)
    bad += int(np.sum(q4k.dequantize(u) != q4k.qdq(x_bits)))
    # byte layout: d, dmin little endian; bit stream; nibble order
    bad += int(np.sum((blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8)) != p["d"]))
    bad += int(np.sum((blocks[..., 2].astype(np.uint16) | (blocks[..., 3].astype(np.uint16) << 8)) != p["dmin"]))
    for idx in np.ndindex(rows, nsb):
        stream = int.from_bytes(bytes(blocks[idx][4:16]), "little")
        for j in range(8):
            bad += int(((stream >> (6 * j)) & 63) != sc_ref[idx][j])
            bad += int(((stream >> (48 + 6 * j)) & 63) != m_ref[idx][j])
        if idx[0] > 3:
            break
    qflat = p["q"].reshape(rows, nsb, 256)
    bad += int(np.sum((blocks[..., 16:] & 15) != qflat[..., 0::2])) + int(np.sum((blocks[..., 16:] >> 4) != qflat[..., 1::2]))
    return bad
