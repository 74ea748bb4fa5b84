"""Pins of the oracle's NVFP4, MXFP4 and Q4_K QDQ and packing.

The checks that recompute every step by an independent route live in
tests/pins.py.  Here they run on the 256x512 workload (N(0, 0.02^2) with 131
N(0, 0.5^2) outliers) and on planted inputs, next to the closed-form and
invariant pins: bits per weight from the project page's "Supported formats"
table, QDQ == dequant(unpack(pack)) ("no extra lossy conversion" on export,
"no requantization" in the QARL weight sync, "Method" section), idempotence,
on-grid outputs and exact-representable round trips.
"""

import json
import os

import numpy as np
import pytest

import workloads
from oracle import nvfp4, mxfp4, q4k
from oracle import primitives as P
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_table.json")
RNG = np.random.default_rng(77)


def _table():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------- closed forms (the table) --
def test_bits_per_weight_matches_table(single):
    t = _table()
    rows, cols = single["W"].shape
    n = rows * cols
    nv = nvfp4.packed_bytes(rows, cols, n_groups=1)
    mx = mxfp4.packed_bytes(rows, cols)
    qk = q4k.packed_bytes(rows, cols)
    assert (nv, mx, qk) == (73_732, 69_632, 73_728)
    assert 8 * (nv - 4) / n == t["NVFP4"]["bits_per_weight"]
    assert 8 * mx / n == t["MXFP4"]["bits_per_weight"]
    assert 8 * qk / n == t["Q4_K"]["bits_per_weight"]
    assert (nvfp4.BLOCK, mxfp4.BLOCK, q4k.SUB, q4k.SUPER) == (
        t["NVFP4"]["block"], t["MXFP4"]["block"], t["Q4_K"]["block"], t["Q4_K"]["super_block"])
    # Q4_K field sizes follow from 4.50 bpw: 4-bit codes, 6+6 bits per sub-block, two fp16 per super-block
    assert 256 * 4 + 8 * (6 + 6) + 2 * 16 == 144 * 8


def test_packed_arrays_have_closed_form_sizes(single):
    W = single["W"]
    s_t = nvfp4.tensor_scale([W])
    c, S = nvfp4.quantize(W, s_t)
    pc, ps = nvfp4.pack(c, S)
    assert pc.nbytes + ps.nbytes + 4 == 73_732
    c, E = mxfp4.quantize(W)
    pc, ps = mxfp4.pack(c, E)
    assert pc.nbytes + ps.nbytes == 69_632
    assert q4k.pack(q4k.quantize(W)).nbytes == 73_728


# ------------------------------------------------------- independent checks --
def test_nvfp4_independent(single):
    W = single["W"]
    s_t = nvfp4.tensor_scale([W])
    assert pins.check_nvfp4_tensor_scale([W]) == 0
    assert pins.check_nvfp4(W, s_t) == 0


def test_mxfp4_independent(single):
    assert pins.check_mxfp4(single["W"]) == 0


def test_q4k_independent(single):
    assert pins.check_q4k(single["W"]) == 0


def _special_bits(rows, cols):
    """bf16 inputs with zeros of both signs, subnormals, huge values and mixed rows."""
    x = RNG.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(RNG.integers(-30, 30, size=(rows, 1))).astype(np.float32)
    b = pins.bf16_torch(x)
    b[0, :] = 0
    b[1, :] = 0x8000                                  # -0.0
    b[2, :] = RNG.integers(1, 0x80, size=cols)        # positive bf16 subnormals
    b[3, :] = RNG.integers(0x8001, 0x8080, size=cols) # negative subnormals
    b[4, :] = RNG.integers(0x7E00, 0x7F7F, size=cols) # very large
    b[5, :16] = 0x3F80                                # one block of 1.0 then zeros
    b[5, 16:] = 0
    return b


def test_formats_on_special_values():
    b = _special_bits(8, 512)
    assert pins.check_mxfp4(b) == 0
    assert pins.check_q4k(b[[0, 1, 2, 3, 5, 6, 7]]) == 0
    for rows in ([0, 1], [2, 3], [5, 6, 7], [6, 7]):
        sub = b[rows]
        assert pins.check_nvfp4(sub, nvfp4.tensor_scale([sub])) == 0


def test_zero_tensor_conventions():
    z = np.zeros((2, 256), np.uint16)
    z[1] = 0x8000
    assert nvfp4.tensor_scale([z]) == np.float32(1.0)
    c, S = nvfp4.quantize(z, nvfp4.tensor_scale([z]))
    assert np.all(S == 0) and np.all(c[0] == 0) and np.all(c[1] == 8)
    assert np.array_equal(nvfp4.qdq(z, 1.0), z)       # signed zeros survive
    c, E = mxfp4.quantize(z)
    assert np.all(E == 0) and np.array_equal(mxfp4.qdq(z), z)
    p = q4k.quantize(z)
    assert np.all(p["d"] == 0) and np.all(p["dmin"] == 0) and np.all(p["q"] == 0)
    assert np.all(P.bf16_to_f32(q4k.qdq(z)) == 0)


# -------------------------------------------------------------- tying ------
def test_nvfp4_tied_group_equals_fused_tensor():
    """QKV as three tensors sharing one scale == the fused QKV matrix."""
    q = pins.bf16_torch(RNG.standard_normal((64, 256)).astype(np.float32) * 0.02)
    k = pins.bf16_torch(RNG.standard_normal((16, 256)).astype(np.float32) * 0.05)
    v = pins.bf16_torch(RNG.standard_normal((16, 256)).astype(np.float32) * 0.01)
    fused = np.concatenate([q, k, v])
    s_sep = nvfp4.tensor_scale([q, k, v])
    assert s_sep == nvfp4.tensor_scale([fused])
    assert pins.check_nvfp4_tensor_scale([q, k, v]) == 0
    sep = np.concatenate([nvfp4.qdq(t, s_sep) for t in (q, k, v)])
    assert np.array_equal(sep, nvfp4.qdq(fused, s_sep))
    # untied V would get its own (smaller) scale and different values
    assert nvfp4.tensor_scale([v]) < s_sep


# ------------------------------------------------------------ on-grid ------
def test_outputs_lie_on_grid(single):
    W = single["W"]
    rows, cols = W.shape
    s_t = nvfp4.tensor_scale([W])
    o = nvfp4.qdq(W, s_t)
    _, S = nvfp4.quantize(W, s_t)
    s = pins.e4m3_val_torch(S)
    grid = pins.bf16_torch(pins.f32(pins.f32(pins.E2M1[None, None, :] * s[..., None]).astype(np.float64) * float(s_t)))
    grid = np.concatenate([grid, grid | 0x8000], axis=-1)          # [rows, blocks, 16]
    ob = o.reshape(rows, cols // 16, 16)
    assert np.all((ob[..., :, None] == grid[..., None, :]).any(axis=-1))
    # MXFP4
    o = mxfp4.qdq(W)
    _, E = mxfp4.quantize(W)
    X = np.ldexp(1.0, E.astype(np.int64) - 127)
    grid = pins.bf16_torch(pins.f32(pins.E2M1[None, None, :] * X[..., None]))
    grid = np.concatenate([grid, grid | 0x8000], axis=-1)
    ob = o.reshape(rows, cols // 32, 32)
    assert np.all((ob[..., :, None] == grid[..., None, :]).any(axis=-1))
    # Q4_K
    o = q4k.qdq(W)
    p = q4k.quantize(W)
    D = pins.f16_val(p["d"])[..., None] * p["sc"]
    M = pins.f16_val(p["dmin"])[..., None] * p["m"]
    grid = pins.bf16_torch(pins.f32(D[..., None] * np.arange(16) - M[..., None]))   # [rows, nsb, 8, 16]
    ob = o.reshape(rows, cols // 256, 8, 32)
    assert np.all((ob[..., :, None] == grid[..., None, :]).any(axis=-1))


# ------------------------------------------------------------ idempotence --
def test_mxfp4_idempotent_exactly(single):
    for b in (single["W"], _special_bits(8, 512)):
        o = mxfp4.qdq(b)
        assert np.array_equal(mxfp4.qdq(o), o)


def test_nvfp4_idempotent_for_normal_block_scales(single):
    W = single["W"]
    s_t = nvfp4.tensor_scale([W])
    o = nvfp4.qdq(W, s_t)
    s_t2 = nvfp4.tensor_scale([o])
    assert s_t2 == s_t                          # the group amax survives QDQ
    _, S = nvfp4.quantize(W, s_t)
    normal = (S >= 8) | (S == 0)                # E4M3 normal or zero scale
    o2 = nvfp4.qdq(o, s_t2)
    rows, cols = W.shape
    same = (o2 == o).reshape(rows, cols // 16, 16).all(axis=-1)
    assert np.all(same[normal])
    # blocks with an E4M3-subnormal scale may move; the workload has none
    assert np.sum(~normal) == 0


def test_q4k_fixed_points(single):
    """Q4_K QDQ is not a projection in general: rounding sc_j to the nearest integer can
    leave the sub-block's top code below 15 (or its bottom code above 0), so a second
    pass sees a narrower range and picks other scales.  What must hold: every sub-block
    whose first-pass codes span 0..15 and whose super-block d and dmin survive the second
    pass is reproduced bit for bit."""
    W = single["W"]
    o = q4k.qdq(W)
    p0, p1 = q4k.quantize(W), q4k.quantize(o)
    o2 = q4k.dequantize(p1)
    rows, cols = W.shape
    q = p0["q"].reshape(rows, cols // 256, 8, 32)
    spans = (q.max(axis=-1) == 15) & (q.min(axis=-1) == 0)
    same_d = ((p0["d"] == p1["d"]) & (p0["dmin"] == p1["dmin"]))[..., None]
    moved = (o != o2).reshape(q.shape).any(axis=-1)
    assert np.sum(moved & spans & same_d) == 0
    assert np.mean(spans & same_d) > 0.5
    assert np.array_equal(p1["sc"][spans & same_d], p0["sc"][spans & same_d])


# ------------------------------------------------- exact-representable trip --
def test_mxfp4_planted_round_trip():
    rows, cols = 4, 256
    codes = RNG.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    E = RNG.integers(100, 140, size=(rows, cols // 32)).astype(np.uint8)
    cb = codes.reshape(rows, -1, 32)
    cb[..., 0] = RNG.choice([6, 7, 14, 15], size=cb.shape[:2])     # each block holds a +-4 or +-6
    x = mxfp4.dequantize(codes, E)
    c2, E2 = mxfp4.quantize(x)
    assert np.array_equal(E2, E)
    # codes agree wherever the value is not a signed zero (-0 and +0 both dequantize to a zero)
    assert np.array_equal(mxfp4.qdq(x), x)
    nz = (codes & 7) != 0
    assert np.array_equal(c2[nz], codes[nz])


def test_nvfp4_planted_round_trip():
    rows, cols = 4, 256
    k = -9
    s_t = np.float32(2.0 ** k)
    codes = RNG.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    S = RNG.integers(8, 0x7E, size=(rows, cols // 16)).astype(np.uint8)   # normal E4M3
    S[0, 0] = 0x7E                                                         # one block at 448
    cb = codes.reshape(rows, -1, 16)
    cb[..., 0] = RNG.choice([7, 15], size=cb.shape[:2])                    # each block holds a +-6
    x = nvfp4.dequantize(codes, S, s_t)
    assert nvfp4.tensor_scale([x]) == s_t
    c2, S2 = nvfp4.quantize(x, s_t)
    assert np.array_equal(S2, S)
    nz = (codes & 7) != 0
    assert np.array_equal(c2[nz], codes[nz])
    assert np.array_equal(nvfp4.qdq(x, s_t), x)


def _sig_bits(n):
    n = abs(int(n))
    while n and n % 2 == 0:
        n //= 2
    return n.bit_length()


def test_q4k_planted_round_trip():
    """Plant d, dmin (powers of two), sc, m and q; synthesize x = bf16(D q - M); then
    qdq(x) == x and quantize(x) reproduces the planted fields.

    Conditions that make this exact: each sub-block holds q = 0 (so min x = -M, exact)
    and q = 15 with 15 D - M exactly representable in bf16 (so max x recovers D); one
    sub-block has sc = 63 and one m = 63 (so d and dmin are recovered); and the bf16
    rounding of every x (at most 2^-8 |x|) stays below D/2, so q is recovered."""
    rows, nsb = 2, 2
    d_val, dmin_val = 2.0 ** -8, 2.0 ** -8
    sc = np.zeros((rows, nsb, 8), np.int64)
    m = np.zeros((rows, nsb, 8), np.int64)
    for idx in np.ndindex(rows, nsb):
        for j in range(8):
            while True:
                s_ = 63 if j == 0 else int(RNG.integers(8, 64))
                m_ = 63 if j == 1 else int(RNG.integers(0, 64))
                if _sig_bits(15 * s_ - m_) <= 8:
                    break
            sc[idx][j], m[idx][j] = s_, m_
    q = RNG.integers(0, 16, size=(rows, nsb, 8, 32))
    q[..., 0] = 0
    q[..., 1] = 15
    vals = (sc[..., None] * q - m[..., None]) * d_val                     # exact in float32
    x = pins.bf16_torch(vals.reshape(rows, nsb * 256).astype(np.float32))
    xv = P.bf16_to_f32(x).astype(np.float64).reshape(q.shape)
    assert np.all(np.abs(xv - vals) < (sc * d_val / 2)[..., None])
    p = q4k.quantize(x)
    assert np.all(pins.f16_val(p["d"]) == d_val) and np.all(pins.f16_val(p["dmin"]) == dmin_val)
    assert np.array_equal(p["sc"], sc) and np.array_equal(p["m"], m)
    assert np.array_equal(p["q"].reshape(q.shape), q)
    assert np.array_equal(q4k.qdq(x), x)
    assert pins.check_q4k(x) == 0


# ------------------------------------------------ brute force on tiny blocks --
def test_block_codes_minimise_squared_error():
    """For fixed block scales, the emitted code vector minimises sum_i (y_i - v(c_i))^2.

    The sum is separable, so the joint minimum is the per-element minimum; check the
    reduction itself on 4-element sub-vectors by enumerating all 16^4 signed code vectors.
    """
    import itertools
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    allv = np.array(list(itertools.product(vals, repeat=4)))              # 65536 x 4
    for _ in range(20):
        y = RNG.standard_normal(4) * 3
        y_b = P.bf16_to_f32(pins.bf16_torch(y.astype(np.float32))).astype(np.float64)
        err = ((allv - y_b) ** 2).sum(axis=1)
        best = allv[np.argmin(err)]
        mags = P.e2m1_encode_mag(np.abs(y_b).astype(np.float32))
        emitted = np.where(np.signbit(y_b), -P.E2M1_MAG[mags], P.E2M1_MAG[mags])
        assert ((emitted - y_b) ** 2).sum() == err.min()
        assert np.allclose(np.abs(best), np.abs(emitted)) or ((best - y_b) ** 2).sum() == err.min()


def test_mxfp4_noclip_rule_by_brute_force(single):
    assert pins.check_mxfp4_noclip(single["W"]) == 0
    assert pins.check_mxfp4_noclip(pins.planted_mx_blocks()) == 0


def test_mxfp4_noclip_never_clips_and_is_minimal():
    """Under noclip every |x| / X is at most 6 (no saturation) unless the block maximum is
    above 6 * 2^125, the top of the last grid bf16 can hold; one exponent lower would put
    the block maximum above 6 unless E is already 0; E differs from the floor rule exactly
    when the maximum's mantissa exceeds 1.5 and the floor rule's E is below 252."""
    b = pins.planted_mx_blocks()
    x = P.bf16_to_f32(b).astype(np.float64)
    a = np.abs(x).max(axis=-1)
    _, E = mxfp4.quantize(b, rule="noclip")
    _, Ef = mxfp4.quantize(b, rule="floor")
    E, Ef = E.astype(np.int64)[:, 0], Ef.astype(np.int64)[:, 0]
    X = np.ldexp(1.0, E - 127)
    top = a > np.ldexp(6.0, 125)
    assert np.all((a / X <= 6.0) | top)
    assert np.all(E[top] == 252) and top.sum() >= 2              # 0x7F7F and 1.75 * 2^127 are planted
    low = np.ldexp(6.0, E - 1 - 127)
    assert np.all((E == 0) | (a > low))
    mant = (b[:, 31] & 0x7F).astype(np.int64)
    normal = ((b[:, 31] >> 7) & 0xFF) >= 1
    want = np.where(normal & (mant > 0x40) & (Ef + 1 <= 252) & (Ef > 0), Ef + 1, Ef)
    ok = normal & (Ef > 0)                                    # above the clamp at E = 0
    assert np.array_equal(E[ok], want[ok])


@pytest.mark.parametrize("rule", ["floor", "noclip"])
def test_mxfp4_every_finite_input_stays_finite(rule):
    """Every finite bf16 value, as the maximum of a block (the other elements a spread of
    smaller values of both signs), gives finite QDQ'd values on the E2M1 grid of the block's
    exponent; in particular the top binade [1.75, 2) * 2^127 must not round up to 2^128."""
    allb = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    finite = allb[(allb & 0x7F80) != 0x7F80]
    blocks = np.zeros((finite.size, 32), np.uint16)
    blocks[:, 0] = finite
    mag = finite & 0x7FFF
    for j in range(1, 32):                                    # smaller magnitudes, alternating signs
        blocks[:, j] = (mag >> (j % 8)) | (0x8000 if j % 2 else 0)
    y = mxfp4.qdq(blocks, rule=rule)
    assert not np.any((y & 0x7F80) == 0x7F80), "a finite input gave Inf or NaN"
    codes, E = mxfp4.quantize(blocks, rule=rule)
    grid = P.bf16_to_f32(y).astype(np.float64) / np.ldexp(1.0, E.astype(np.int64) - 127)
    assert np.all(np.isin(np.abs(grid), pins.E2M1))
    planted = np.array([[0x7F60] + [0x3F80] * 31, [0x7F7F] + [0xFF70] * 31, [0x7F70] * 32], np.uint16)
    yp = P.bf16_to_f32(mxfp4.qdq(planted, rule=rule)).astype(np.float64)
    assert np.all(np.isfinite(yp)) and np.abs(yp).max() == np.ldexp(6.0, 125)