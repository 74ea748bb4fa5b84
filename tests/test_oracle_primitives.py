"""Pins of the oracle's number-format primitives against independent routines.

Each primitive is checked against something other than itself: torch's own
casts (bfloat16, float8_e4m3fn, float8_e8m0fnu), Python's struct half-float
packing, or a brute-force nearest search written with exact float64 distances.
"""

import struct

import numpy as np
import pytest
import torch

from oracle import primitives as P

RNG = np.random.default_rng(1234)


def _torch_bf16_bits(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _finite_f32_sample(n):
    b = RNG.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = b.view(np.float32)
    return x[np.isfinite(x)]


def test_bf16_widen_is_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = P.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_bf16_narrow_matches_torch_rne():
    x = _finite_f32_sample(400_000)
    # bf16 overflow only for |x| > bf16 max; keep finite results (the method never overflows)
    x = x[np.abs(x) < np.float32(3.38e38)]
    # every exact midpoint and its neighbours, for even and odd kept patterns
    hi = RNG.integers(0, 0x7F7F, size=20_000, dtype=np.uint32)
    mids = ((hi << 16) | 0x8000).view(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    x = np.concatenate([x, near, -near, np.float32([0.0, -0.0, 1e-45, -1e-45, 1.0])])
    assert np.array_equal(P.f32_to_bf16(x), _torch_bf16_bits(x))


def _f16_bruteforce(x):
    """Nearest finite binary16 to each x (exact float64 distances), ties to the even pattern,
    saturating at +-65504."""
    pats = np.arange(0x7C00, dtype=np.uint16)                # non-negative finite patterns
    vals = pats.view(np.float16).astype(np.float64)
    out = np.empty(x.shape, np.uint16)
    for i, xi in enumerate(np.asarray(x, np.float64)):
        a = abs(xi)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        p = pats[best[0]] if best.size == 1 else pats[best[(pats[best] & 1) == 0][0]]
        out[i] = p | (0x8000 if np.signbit(xi) else 0)
    return out


def test_f16_against_bruteforce_and_struct():
    xs = [RNG.standard_normal(300).astype(np.float32) * s for s in (1e-7, 1e-5, 1e-3, 1.0, 1e3, 3e4)]
    mids = (np.arange(0, 0x7BFF, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
            + np.arange(1, 0x7C00, 97, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2
    x = np.concatenate(xs + [mids.astype(np.float32), np.float32([0.0, -0.0, 65504, 65519.9, 65520, 7e4, -1e9])])
    got = P.f32_to_f16_bits(x)
    assert np.array_equal(got, _f16_bruteforce(x))
    for xi, gi in zip(x[:500], got[:500]):                   # python's own half packing (RNE)
        assert struct.unpack("<H", struct.pack("<e", float(xi)))[0] == gi


def _nearest_bruteforce(u, mags):
    """argmin_i |u - mags[i]|, ties to the even index, on exact float64 distances.

    Inputs above 2^40 are lowered to 2^40 first: beyond the largest magnitude the
    largest magnitude is the unique nearest entry either way, and below 2^40 every
    float32 input minus a table entry is exact in float64.
    """
    u = np.minimum(np.asarray(u, np.float64), 2.0 ** 40)[:, None]
    dist = np.abs(u - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    ismin = dist == best
    idx = np.arange(mags.size)[None, :]
    # lowest even index among the minima if any, else the single minimum
    even = np.where(ismin & (idx % 2 == 0), idx, 10 ** 6).min(axis=1)
    anyidx = np.where(ismin, idx, 10 ** 6).min(axis=1)
    return np.where(ismin.sum(axis=1) > 1, even, anyidx).astype(np.uint8)


def test_e2m1_encode_bruteforce_all_bf16():
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)  # all non-negative finite bf16
    y = P.bf16_to_f32(bits)
    assert np.array_equal(P.e2m1_encode_mag(y), _nearest_bruteforce(y, P.E2M1_MAG))


def test_e2m1_thresholds_and_ties():
    # threshold value -> code it must take (the tie goes to the even code), and just above it
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for t, code in cases:
        assert P.e2m1_encode_mag(np.float32([t]))[0] == code
        above = np.nextafter(np.float32(t), np.float32(np.inf))
        below = np.nextafter(np.float32(t), np.float32(0))
        # strictly inside the intervals the result is unambiguous
        assert P.e2m1_encode_mag(np.float32([below]))[0] == _nearest_bruteforce([below], P.E2M1_MAG)[0]
        assert P.e2m1_encode_mag(np.float32([above]))[0] == _nearest_bruteforce([above], P.E2M1_MAG)[0]
    assert list(P.e2m1_encode_mag(np.float32([0, 0.5, 1, 1.5, 2, 3, 4, 6, 7, 1e30, np.inf]))) == \
        [0, 1, 2, 3, 4, 5, 6, 7, 7, 7, 7]
    assert P.e2m1_encode_mag(np.float32([np.nan]))[0] == 0
    assert list(P.e2m1_value(np.arange(16, dtype=np.uint8))) == \
        [0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6]


def _torch_e4m3_code(u):
    t = torch.from_numpy(np.minimum(np.asarray(u, np.float32), np.float32(448.0)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_table():
    assert P.E4M3_POS.size == 127
    assert P.E4M3_POS[0x7E] == 448.0 and P.E4M3_POS[1] == 2.0 ** -9 and P.E4M3_POS[8] == 2.0 ** -6
    assert np.all(np.diff(P.E4M3_POS) > 0)
    # decode agrees with torch's float8_e4m3fn for every finite non-negative code
    codes = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(P.e4m3_value(codes), ref)


def test_e4m3_encode_all_bf16_and_midpoints():
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    u = P.bf16_to_f32(bits)
    mids = ((P.E4M3_POS[:-1] + P.E4M3_POS[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    u = np.concatenate([u, mids, up, dn, np.float32([448, 448.0001, 463.99, 464, 465, 1e30])])
    got = P.e4m3_encode(u)
    assert np.array_equal(got, _torch_e4m3_code(u))
    assert np.array_equal(got, _nearest_bruteforce(u, P.E4M3_POS))
    assert P.e4m3_encode(np.float32([1e30]))[0] == 0x7E


def test_e8m0_decode_against_torch():
    E = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(E.copy()).view(torch.float8_e8m0fnu).float().numpy()
    assert np.array_equal(P.e8m0_value(E).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("k", range(-140, 128, 7))
def test_floor_log2_exact(k):
    p = np.ldexp(1.0, k)
    assert P.floor_log2(np.float64([p]))[0] == k
    assert P.floor_log2(np.float64([np.nextafter(p, 0)]))[0] == k - 1
    assert P.floor_log2(np.float64([p * 1.999]))[0] == k
