"""Planted mistakes in the oracle must fail a pin.

Each test swaps one oracle function for a plausible wrong version (on the CPU,
with pytest's monkeypatch) and checks that the independent pins of
tests/pins.py, or the primitive brute-force checks, report violations.  This
is what makes the pins evidence: they would notice a dropped term, a wrong
tie rule, a wrong constant, a transposed operand or a swapped nibble.
"""

import numpy as np

import workloads
from oracle import primitives as P
from oracle import nvfp4, mxfp4, q4k, lora
from tests import pins
from tests.test_oracle_primitives import _nearest_bruteforce


def _w():
    return workloads.single_256x512()["W"]


def test_mutation_e2m1_ties_away_is_caught(monkeypatch):
    def ties_away(y):
        y = np.asarray(y, np.float64)
        mid = (P.E2M1_MAG[:-1] + P.E2M1_MAG[1:]) / 2
        return np.searchsorted(mid, y, side="right").astype(np.uint8)   # ties go up
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    y = P.bf16_to_f32(bits)
    assert np.any(ties_away(y) != _nearest_bruteforce(y, P.E2M1_MAG))
    monkeypatch.setattr(nvfp4, "e2m1_encode_mag", ties_away)
    monkeypatch.setattr(mxfp4, "e2m1_encode_mag", ties_away)
    W = _w()
    # MXFP4 scaled values are exact, so ties (0.25, 0.75, ...) do occur on this data
    assert pins.check_mxfp4(W) > 0


def test_mutation_wrong_tensor_divisor_is_caught(monkeypatch):
    monkeypatch.setattr(nvfp4, "TENSOR_DIV", np.float32(2560.0))
    assert pins.check_nvfp4_tensor_scale([_w()]) > 0


def test_mutation_nvfp4_dequant_order_is_caught(monkeypatch):
    """fl(v * fl(s * s_t)) instead of fl(fl(v * s) * s_t): the two differ after the bf16
    rounding for about 0.2% of (tensor scale, block scale) pairs; plant such pairs."""
    def reordered(codes, S, s_t):
        rows, cols = codes.shape
        c = codes.reshape(rows, cols // 16, 16)
        v = P.E2M1_MAG[c & 7].astype(np.float32)
        ss = (P.e4m3_value(S) * np.float32(s_t)).astype(np.float32)[..., None]
        o = (v * ss).astype(np.float32)
        bits = P.f32_to_bf16(o) | ((c >> 3).astype(np.uint16) << np.uint16(15))
        return bits.reshape(rows, cols)
    A = P.bf16_to_f32(np.arange(0x3000, 0x4000, dtype=np.uint32).astype(np.uint16))
    st = (A / np.float32(2688)).astype(np.float32)
    s = P.e4m3_value(np.arange(1, 127, dtype=np.uint8))
    o1 = ((np.float32(1.5) * s)[None, :] * st[:, None]).astype(np.float32)
    o2 = (np.float32(1.5) * (s[None, :] * st[:, None]).astype(np.float32)).astype(np.float32)
    i, j = np.argwhere(P.f32_to_bf16(o1) != P.f32_to_bf16(o2))[0]
    codes = np.full((1, 16), 3, np.uint8)                      # magnitude 1.5
    S = np.array([[j + 1]], np.uint8)
    assert pins.check_nvfp4_dequant(codes, S, st[i]) == 0
    monkeypatch.setattr(nvfp4, "dequantize", reordered)
    assert pins.check_nvfp4_dequant(codes, S, st[i]) > 0


def test_mutation_e4m3_ties_up_is_caught(monkeypatch):
    def e4m3_no_tie_even(u):
        # round half up instead of half to even
        u = np.asarray(u, np.float64)
        mid = (P.E4M3_POS[:-1] + P.E4M3_POS[1:]) / 2
        return np.searchsorted(mid, u, side="right").astype(np.uint8)
    monkeypatch.setattr(nvfp4, "e4m3_encode", e4m3_no_tie_even)
    # plant block maxima that land exactly on E4M3 midpoints: a = u * 6 * s_t with s_t = 1
    mids = ((P.E4M3_POS[8:40] + P.E4M3_POS[9:41]) / 2)
    x = np.zeros((1, 16 * mids.size), np.float32)
    x[0, ::16] = (mids * 6).astype(np.float32)
    x[0, 16 * (mids.size - 1) + 1] = 2688.0                 # group amax 2688 -> s_t = 1
    xb = pins.bf16_torch(x)
    assert pins.check_nvfp4(xb, nvfp4.tensor_scale([xb])) > 0


def test_mutation_mxfp4_ceil_rule_is_caught(monkeypatch):
    def ceil_rule(x_bits, rule="floor"):
        x_bits = np.asarray(x_bits, np.uint16)
        rows, cols = x_bits.shape
        x = P.bf16_to_f32(x_bits).reshape(rows, cols // 32, 32)
        a = np.abs(x).max(axis=-1)
        e = np.ceil(np.log2(np.maximum(a, 1e-38) / 6.0)).astype(np.int64)
        E = np.where(a > 0, np.clip(e + 127, 0, 254), 0)
        X = P.e8m0_value(E)
        y = (np.abs(x) / X[..., None]).astype(np.float32)
        codes = (np.signbit(x).astype(np.uint8) << 3) | P.e2m1_encode_mag(y)
        return codes.reshape(rows, cols), E.astype(np.uint8)
    monkeypatch.setattr(mxfp4, "quantize", ceil_rule)
    assert pins.check_mxfp4(_w()) > 0


def test_mutation_q4k_unclamped_min_is_caught(monkeypatch):
    orig = q4k.quantize

    def unclamped(x_bits, rule="minmax"):
        # shift every input up so a block is all-positive, then quantize as if min were not clamped
        p = orig(x_bits, rule)
        x = P.bf16_to_f32(x_bits).reshape(p["sc"].shape + (32,))
        allpos = (x.min(axis=-1) > 0)
        p["m"] = np.where(allpos, 1, p["m"]).astype(np.uint8)
        return p
    x = pins.bf16_torch(np.abs(np.random.default_rng(3).standard_normal((2, 512))).astype(np.float32) + 0.5)
    assert pins.check_q4k(x) == 0
    monkeypatch.setattr(q4k, "quantize", unclamped)
    assert pins.check_q4k(x) > 0


def test_mutation_q4k_nibble_swap_is_caught(monkeypatch):
    orig = q4k.pack

    def swapped(p):
        b = orig(p)
        b[..., 16:] = ((b[..., 16:] & 15) << 4) | (b[..., 16:] >> 4)
        return b
    monkeypatch.setattr(q4k, "pack", swapped)
    assert pins.check_q4k(_w()[:8]) > 0


def test_mutation_nvfp4_sign_dropped_for_zero_codes_is_caught(monkeypatch):
    orig = nvfp4.quantize

    def dropsign(x_bits, s_t):
        c, S = orig(x_bits, s_t)
        c = np.where((c & 7) == 0, 0, c).astype(np.uint8)
        return c, S
    monkeypatch.setattr(nvfp4, "quantize", dropsign)
    W = _w()
    assert pins.check_nvfp4(W, nvfp4.tensor_scale([W])) > 0


def test_mutation_lora_descending_order_is_caught(monkeypatch):
    def descending(W_bits, A_bits, B_bits):
        W, A, B = P.bf16_to_f32(W_bits), P.bf16_to_f32(A_bits), P.bf16_to_f32(B_bits)
        acc = np.zeros(W.shape, np.float32)
        for k in reversed(range(A.shape[0])):
            acc = (acc + (B[:, k:k + 1] * A[k:k + 1, :]).astype(np.float32)).astype(np.float32)
        return P.f32_to_bf16((W + acc).astype(np.float32))
    monkeypatch.setattr(lora, "merge", descending)
    from tests.test_oracle_misc import test_lora_merge_order_is_ascending_k
    try:
        test_lora_merge_order_is_ascending_k()
    except AssertionError:
        return
    raise AssertionError("descending merge order was not caught")


def test_mutation_noclip_uncapped_exponent_is_caught(monkeypatch):
    """The noclip rule clamped at E = 254 instead of 252 sends block maxima in
    [1.75, 2) * 2^127 to 2^128 (Inf); the brute-force exponent pin notices it."""
    monkeypatch.setattr(mxfp4, "NOCLIP_E_MAX", 254)
    assert pins.check_mxfp4_noclip(pins.planted_mx_blocks()) > 0


def test_mutation_q4k_mse_index_order_is_caught(monkeypatch):
    """The mse rule's scores summed over all 32 elements in index order instead of the stated
    tree: the planted near ties decide differently, and their pin fails."""
    F = np.float32

    def index_order(x, mn, mx):
        base = ((mx - mn).astype(F) / F(15.0)).astype(F)
        t = (x - mn[..., None]).astype(F)
        errs, scales = [], []
        for k in range(q4k.MSE_CANDIDATES):
            s = (base * F(1.0 - k / 16.0)).astype(F)
            zero = s == 0
            with np.errstate(divide="ignore"):
                r = np.where(zero, F(0.0), F(1.0) / np.where(zero, F(1.0), s)).astype(F)
            q = np.clip(P.rint((t * r[..., None]).astype(F)), 0, 15).astype(F)
            e = (((q * s[..., None]).astype(F) + mn[..., None]).astype(F) - x).astype(F)
            sq = (e * e).astype(F)
            acc = sq[..., 0]
            for i in range(1, sq.shape[-1]):
                acc = (acc + sq[..., i]).astype(F)
            errs.append(acc)
            scales.append(s)
        err = np.stack(errs, -1)
        best = np.argmin(err, -1)
        scale = np.take_along_axis(np.stack(scales, -1), best[..., None], -1)[..., 0]
        return scale.astype(F), err, best

    from tests.test_oracle_q4k_mse import test_near_ties_follow_the_stated_order
    test_near_ties_follow_the_stated_order()
    monkeypatch.setattr(q4k, "mse_scale", index_order)
    try:
        test_near_ties_follow_the_stated_order()
    except AssertionError:
        return
    raise AssertionError("the index summation order was not caught")
