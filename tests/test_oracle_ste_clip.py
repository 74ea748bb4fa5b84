"""Pins of the oracle's saturation masks and clipped STE (CPU).

What pins them, independent of the mask code:
- MXFP4: y = |x| / 2^(E-127) is exact, so an element saturates exactly when |x| > 6 * 2^(E-127)
  in float64 arithmetic, with E taken from the scale bytes quantize() returns;
- MXFP4 under the noclip rule: no element saturates (the rule's definition);
- MXFP4 floor rule: planted block maxima just above and at 6 * 2^(E-127) saturate / do not;
- NVFP4: a saturated element carries the largest magnitude code (7); outside a narrow band
  around 6 d (d = s * s_t, exact in float64) the mask is fixed by the exact comparison of |x|
  with 6 d, so a rounding slip can only matter within 1e-6 of the boundary;
- the clipped STE equals the identity STE where nothing saturates and is +0.0 (or adds +0.0)
  where something does.
"""

import numpy as np

import workloads
from oracle import mxfp4, nvfp4, ste
from oracle import primitives as P

RNG = np.random.default_rng(77)


def _x():
    return workloads.single_256x512()["W"]


def test_mxfp4_mask_is_the_exact_comparison():
    x = _x()
    for rule in ("floor", "noclip"):
        _, E = mxfp4.quantize(x, rule)
        lim = np.ldexp(6.0, E.astype(np.int64) - 127)                  # float64, exact
        ax = np.abs(P.bf16_to_f32(x).astype(np.float64)).reshape(x.shape[0], -1, 32)
        want = (ax > lim[..., None]).reshape(x.shape)
        got = mxfp4.saturated(x, rule)
        assert np.array_equal(got, want), rule
    assert not mxfp4.saturated(x, "noclip").any()
    assert mxfp4.saturated(x, "floor").sum() > 0                       # the workload has such blocks


def test_mxfp4_planted_maxima():
    x = np.zeros((4, 64), np.float32)
    # block maxima in [4, 8): E - 127 = floor(log2 max) - 2 = 0, so X = 1 and the limit is 6
    x[0, :32] = 0.5
    x[0, 5] = 7.0          # 7 = 1.75 * 4: E - 127 = 0, 6X = 6 < 7: saturates
    x[0, 6] = 6.0          # on the grid: not saturated
    x[1, :32] = 0.5
    x[1, 3] = 6.0          # significand 1.5: 6X = 6 exactly, nothing saturates
    x[2, 32:] = -0.25
    x[2, 40] = -7.5        # 1.875 * 4: saturates
    x[2, 41] = -6.5        # also above 6X = 6
    x[3, 32] = 5.0         # significand 1.25: nothing saturates
    bits = P.f32_to_bf16(x)
    m = mxfp4.saturated(bits)
    want = np.zeros_like(m)
    want[0, 5] = want[2, 40] = want[2, 41] = True
    assert np.array_equal(m, want)
    assert not mxfp4.saturated(bits, "noclip").any()


def test_nvfp4_mask_against_exact_boundary():
    for x, s_t in ((_x(), None), (_x(), np.float32(1e-5)),
                   (P.f32_to_bf16(RNG.standard_t(3, size=(96, 256)).astype(np.float32)), None)):
        s_t = nvfp4.tensor_scale([x]) if s_t is None else s_t
        codes, S = nvfp4.quantize(x, s_t)
        m = nvfp4.saturated(x, s_t)
        assert np.all((codes[m] & 7) == 7)                              # saturated -> top code
        d = (P.e4m3_value(S).astype(np.float64) * np.float64(s_t))      # exact product
        ax = np.abs(P.bf16_to_f32(x).astype(np.float64)).reshape(x.shape[0], -1, 16)
        ratio = (ax / np.where(d == 0, np.inf, d)[..., None]).reshape(x.shape)
        clear = np.abs(ratio - 6.0) > 6e-6
        assert np.array_equal(m[clear], (ratio > 6.0)[clear])
    # a tensor scale far below the data's: almost every block saturates at the E4M3 maximum
    x = _x()
    m = nvfp4.saturated(x, np.float32(1e-6))
    assert m.mean() > 0.5


def test_nvfp4_zero_and_tiny_blocks():
    x = np.zeros((2, 32), np.float32)
    x[0, :16] = 1e-30                        # u rounds to E4M3 0: d == 0, nothing saturates
    x[1, 16:] = 3.0
    bits = P.f32_to_bf16(x)
    assert not nvfp4.saturated(bits, np.float32(1.0)).any()


def test_clipped_ste():
    x = _x()
    g = P.f32_to_bf16(RNG.standard_normal(x.shape).astype(np.float32))
    m = mxfp4.saturated(x)
    out = ste.ste_backward_clipped(g, m)
    plain = ste.ste_backward(g)
    assert np.array_equal(out[~m], plain[~m])
    assert np.all(out[m].view(np.uint32) == 0)                           # +0.0
    none = ste.ste_backward_clipped(g, np.zeros_like(m))
    assert np.array_equal(none.view(np.uint32), plain.view(np.uint32))
    acc = np.full(x.shape, -0.0, np.float32)
    acc2 = ste.ste_backward_clipped(g, m, acc, accumulate=True)
    assert np.all(acc2[m].view(np.uint32) == 0)                          # -0.0 + +0.0 = +0.0
    assert np.array_equal(acc2[~m], (acc[~m].astype(np.float64) + plain[~m]).astype(np.float32))
