"""Pins of the oracle's Q4_K "mse" sub-block scale rule (CPU).

Independent of the rule's float32 code, they check what it must achieve and its special cases:
- the chosen candidate minimizes the sub-block's squared error recomputed in float64 from the
  candidate scales (within float32 summation noise), so a wrong index, a reversed comparison or
  a dropped term fails;
- k = 0 is the min/max rule, so the chosen error is never above the min/max scale's;
- sub-blocks that already sit on the min/max grid (error 0 at k = 0) and constant sub-blocks
  keep the min/max scale;
- with every sub-block on k = 0 the whole quantizer equals the min/max rule;
- near ties, where the float32 summation order decides between two candidates: planted
  sub-blocks on which summing in plain index order would choose differently are decided by
  the stated order (quarters of 8 in index order, then (q0 + q1) + (q2 + q3)), against a
  scalar emulation of that order with one float32 rounding per operation.
"""

import json
import os
import struct

import numpy as np

import workloads
from oracle import q4k
from oracle import primitives as P

RNG = np.random.default_rng(2718)


def _extremes(x):
    mn = np.minimum(np.min(x, axis=-1), np.float32(0.0))
    mn = np.where(mn == 0, np.float32(0.0), mn).astype(np.float32)
    mx = np.max(x, axis=-1)
    mx = np.where(mx == 0, np.float32(0.0), mx).astype(np.float32)
    return mn, mx


def _err64(x, mn, s):
    """Squared error of the sub-blocks under scale s (float64 arithmetic, ties to even)."""
    x64, mn64, s64 = x.astype(np.float64), mn.astype(np.float64)[..., None], s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s64 == 0, 0.0, np.clip(np.rint((x64 - mn64) / np.where(s64 == 0, 1.0, s64)), 0, 15))
    return ((q * s64 + mn64 - x64) ** 2).sum(axis=-1)


def _subblocks(bits):
    rows, cols = bits.shape
    return P.bf16_to_f32(bits).reshape(rows, cols // 256, 8, 32)


def test_choice_minimizes_float64_error():
    for bits in (workloads.single_256x512()["W"],
                 P.f32_to_bf16((RNG.standard_t(2, size=(64, 512)) * 0.02 + 0.001).astype(np.float32))):
        x = _subblocks(bits)
        mn, mx = _extremes(x)
        scale, err32, best = q4k.mse_scale(x, mn, mx)
        base = ((mx - mn).astype(np.float32) / np.float32(15.0)).astype(np.float32)
        e64 = np.stack([_err64(x, mn, (base * np.float32(1 - k / 16)).astype(np.float32)) for k in range(8)], -1)
        chosen = np.take_along_axis(e64, best[..., None], -1)[..., 0]
        tol = 1e-5 * e64.min(-1) + 1e-30
        assert np.all(chosen <= e64.min(-1) + tol)
        assert np.all(chosen <= e64[..., 0] + tol)                     # never worse than min/max
        assert (best > 0).mean() > 0.05                                # the search does act
        assert np.allclose(err32, e64, rtol=1e-5, atol=1e-30)


def test_special_cases():
    x = np.zeros((1, 1, 8, 32), np.float32)
    base = np.float32(0.25)
    x[0, 0, 0] = (np.float32(-1.0) + base * np.arange(16, dtype=np.float32).repeat(2)).astype(np.float32)  # on the grid
    x[0, 0, 1] = 0.5                                                    # constant (mn clamps to 0)
    x[0, 0, 2] = 0.0                                                    # all zero
    mn, mx = _extremes(x)
    scale, _, best = q4k.mse_scale(x, mn, mx)
    assert best[0, 0, 0] == 0 and best[0, 0, 1] == 0 and best[0, 0, 2] == 0


def test_equal_to_minmax_when_nothing_shrinks():
    # every sub-block on its own min/max grid: the mse rule reproduces the min/max quantizer
    rows = 8
    lo = -(RNG.integers(1, 8, size=(rows, 2, 8, 1)).astype(np.float32) * np.float32(0.125))
    step = RNG.integers(1, 4, size=(rows, 2, 8, 1)).astype(np.float32) * np.float32(0.0625)
    lvl = np.stack([RNG.permutation(np.arange(16).repeat(2)) for _ in range(rows * 16)]).reshape(rows, 2, 8, 32)
    x = (lo + step * lvl.astype(np.float32)).astype(np.float32).reshape(rows, 512)
    bits = P.f32_to_bf16(x)
    assert np.array_equal(P.bf16_to_f32(bits), x)                        # exactly representable
    a, b = q4k.quantize(bits), q4k.quantize(bits, "mse")
    for key in ("d", "dmin", "sc", "m", "q"):
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------- near ties ----
NEAR_TIES = os.path.join(os.path.dirname(__file__), "golden", "q4k_mse_near_ties.json")


def _f32(v):
    """One float32 rounding of a Python float (struct: IEEE RNE)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _scores_scalar(xs, order):
    """Scalar Python emulation of the candidates' float32 scores: every +, -, *, / is done
    in double and rounded once to float32 (exact for one operation on float32 operands),
    rint is Python's round (half to even).  order: "stated" (quarters of 8 in index order,
    then (q0 + q1) + (q2 + q3)) or "index" (all 32 in index order)."""
    mn = min(min(xs), 0.0)
    mx = max(xs)
    base = _f32(_f32(mx - mn) / 15.0)
    out = []
    for k in range(8):
        s = _f32(base * (1.0 - k / 16.0))
        r = _f32(1.0 / s)
        sq = []
        for x in xs:
            q = min(max(round(_f32(_f32(x - mn) * r)), 0), 15)
            e = _f32(_f32(_f32(q * s) + mn) - x)
            sq.append(_f32(e * e))
        if order == "stated":
            parts = []
            for j in range(4):
                acc = sq[8 * j]
                for i in range(1, 8):
                    acc = _f32(acc + sq[8 * j + i])
                parts.append(acc)
            out.append(_f32(_f32(parts[0] + parts[1]) + _f32(parts[2] + parts[3])))
        else:
            acc = sq[0]
            for i in range(1, 32):
                acc = _f32(acc + sq[i])
            out.append(acc)
    return out


def _first_min(v):
    return min(range(len(v)), key=lambda k: (v[k], k))


def test_near_ties_follow_the_stated_order():
    """Planted sub-blocks (found by the search in tests/golden/q4k_mse_near_ties.py, inputs
    only) whose two best candidates lie within float32 rounding of each other, so that the
    summation order decides: the index-order sum picks another candidate than the stated
    order.  The oracle must pick the stated order's candidate."""
    with open(NEAR_TIES) as f:
        blocks = np.array(json.load(f)["subblocks_bf16_bits"], np.uint16)
    assert blocks.shape[0] >= 2 and blocks.shape[1] == 32
    for blk in blocks:
        xs = [float(v) for v in P.bf16_to_f32(blk)]
        stated, index = _scores_scalar(xs, "stated"), _scores_scalar(xs, "index")
        assert _first_min(stated) != _first_min(index)             # the order decides here
        x = np.zeros((1, 1, 8, 32), np.float32)
        x[0, 0, 3] = P.bf16_to_f32(blk)
        mn, mx = _extremes(x)
        _, err, best = q4k.mse_scale(x, mn, mx)
        assert best[0, 0, 3] == _first_min(stated)
        assert np.array_equal(err[0, 0, 3].astype(np.float64), np.array(stated))
