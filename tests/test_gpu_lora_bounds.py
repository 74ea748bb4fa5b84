"""GPU parity: the merged weight's tensor scale when pass 1 keeps no M.

Without an M scratch, launches large enough for 32-row units take a maximum pass that
merges exactly only the elements that a bound on |B.A| says could reach the running
maximum; each case here shares its launch with a large filler matrix so that it runs that
pass (checked through the layout query).  These cases are built so that a wrong or
too tight bound would change the result: the maximum of M sits where |W| is not the
largest (the adapter decides it), the largest |W| is cancelled by the adapter, the
maximum lies in the last row and column, values reach below fp32's normal range, and
W, A or B hold an infinity or a NaN.  Each is compared with the oracle's tensor scale of
the fully merged M (bits, or NaN for NaN), and with the pass that stores M.
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
from oracle import lora, nvfp4
from oracle import primitives as P
from tests.gpu_util import dev, f32bits

pytestmark = pytest.mark.gpu


def _bits(x):
    return P.f32_to_bf16(np.asarray(x, np.float32))


def _case(rows, cols, r, seed, w=0.02, a=0.01, b=0.001):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * w, rng.standard_normal((r, cols)) * a,
            rng.standard_normal((rows, r)) * b)


_FILLER = {}


def _filler():
    """A 4096 x 16384 matrix with zero adapters (M = W) in a group of its own: with it a
    launch is large enough for 32-row units, the layout whose pass 1 without M merges
    only where the bound requires (smaller launches take the matrix-core pass)."""
    if not _FILLER:
        g = torch.Generator(device="cuda").manual_seed(77)
        W = (torch.randn((4096, 16384), generator=g, device="cuda") * 0.02).bfloat16()
        _FILLER.update(W=W, A=torch.zeros((16, 16384), dtype=torch.bfloat16, device="cuda"),
                       B=torch.zeros((4096, 16), dtype=torch.bfloat16, device="cuda"),
                       s=np.float32(W.float().abs().max().item()) / np.float32(2688.0))   # IEEE on the host
    return _FILLER


def _with_filler(items):
    f = _filler()
    out = items + [dict(W=f["W"], A=f["A"], B=f["B"], group=max(it["group"] for it in items) + 1, M=None)]
    if all(it.get("M") is None for it in items):
        assert fq.qf_lora_layout(out)[4] == 32, "the launch must run 32-row units"
    return out


def _scales(cases, with_M):
    items = []
    for g, (W, A, B) in enumerate(cases):
        rows, cols = W.shape
        items.append(dict(W=dev(W), A=dev(A), B=dev(B), group=g,
                          M=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") if with_M else None))
    items = _with_filler(items)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = fq.qf_lora_merge_tensor_scale_nvfp4_grouped(items, len(items), d_nonfinite=flag)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    assert f32bits(s[-1]) == f32bits(np.float32(_filler()["s"])), "filler matrix"
    return s[:-1], int(flag.item())


def _check(cases, what):
    """cases: list of (W, A, B) bf16 bit arrays, one tied group each."""
    want, bad = [], False
    for W, A, B in cases:
        M = lora.merge(W, A, B)
        want.append(nvfp4.tensor_scale([M]))
        bad = bad or nvfp4.group_amax([M])[1]
    for with_M in (False, True):
        got, flag = _scales(cases, with_M)
        for g, (x, y) in enumerate(zip(got, want)):
            if np.isnan(y):
                assert np.isnan(x), f"{what} (M kept: {with_M}) group {g}: {x} for NaN"
            else:
                assert f32bits(x) == f32bits(y), f"{what} (M kept: {with_M}) group {g}: {x!r} != {y!r}"
        assert flag == int(bad), f"{what} (M kept: {with_M}): non-finite flag {flag}"


def _bf(x):
    return _bits(np.asarray(x, np.float32))


def test_adapter_decides_the_maximum():
    """|W| is largest at (0, 0), but B.A lifts a small-|W| element in the last row and
    column above it; a second matrix has the same in its first row, last column."""
    cases = []
    for i, (rows, cols, r) in enumerate([(100, 1056, 16), (67, 544, 7)]):
        W, A, B = _case(rows, cols, r, seed=7 + i, a=0.001, b=0.001)
        W[0, 0] = 0.09
        p, q = (rows - 1, cols - 1) if i == 0 else (0, cols - 1)
        A[:, q] = 0.3
        B[p, :] = 0.05                  # S[p, q] = r * 0.015
        cases.append((_bf(W), _bf(A), _bf(B)))
    _check(cases, "adapter decides")


def test_cancelled_largest_weight():
    """The largest |W| is cancelled by the adapter; the maximum of M is the second
    largest |W| plus a small positive adapter term, late in the matrix."""
    rows, cols, r = 96, 1024, 16
    W, A, B = _case(rows, cols, r, seed=3, w=0.01, a=0.0, b=0.0)
    W[1, 5] = 0.1
    A[:, 5] = 0.25
    B[1, :] = -0.0125                   # S[1, 5] = -0.05: M[1, 5] = 0.05
    W[90, 1000] = 0.08
    A[:, 1000] = 0.01
    B[90, :] = 0.01                     # M[90, 1000] = 0.0816
    _check([(_bf(W), _bf(A), _bf(B))], "cancelled maximum")


def test_single_rank_and_ragged_tail():
    """Rank 1, 33 rows (a partial 32-row unit) and a partial 512-column slab."""
    W, A, B = _case(33, 544, 1, seed=11, a=0.2, b=0.2)
    _check([(_bf(W), _bf(A), _bf(B))], "rank 1 ragged")


def test_below_normal_range():
    """W, A and B near and below fp32's smallest normal: the adapter's products are
    subnormal or flush to zero in fp32, and the bound's absolute slack must cover them."""
    W, A, B = _case(64, 512, 16, seed=5, w=1e-38, a=1e-20, b=1e-19)
    W[40, 300] = 3e-38
    _check([(_bf(W), _bf(A), _bf(B))], "tiny values")


def test_zero_weights_and_adapters():
    z = np.zeros((32, 512), np.uint16)
    _check([(z, np.zeros((16, 512), np.uint16), np.zeros((32, 16), np.uint16))], "all zero")


@pytest.mark.parametrize("where", ["W_nan", "W_inf", "A_inf", "B_nan", "A_inf_B_zero_row"])
def test_nonfinite_inputs(where):
    W, A, B = _case(80, 1024, 16, seed=23)
    W, A, B = _bf(W), _bf(A), _bf(B)
    if where == "W_nan":
        W[77, 1001] = 0x7FC1
    elif where == "W_inf":
        W[5, 700] = 0xFF80               # -inf
    elif where == "A_inf":
        A[3, 640] = 0x7F80
    elif where == "B_nan":
        B[70, 2] = 0x7FC0
    else:                               # inf x 0 = NaN in every row whose B[:, 9] is 0
        A[9, 17] = 0x7F80
        B[:, 9] = 0
    _check([(W, A, B)], where)


def test_many_groups_one_launch():
    """15 descriptors (and the filler) in one launch, 5 tied groups, the maxima spread over
    different descriptors."""
    cases, groups = [], []
    for i in range(15):
        W, A, B = _case(48 + 7 * i, 512 + 32 * (i % 4), 1 + (i * 5) % 16, seed=100 + i, a=0.05, b=0.05)
        cases.append((_bf(W), _bf(A), _bf(B)))
        groups.append(i % 5)
    items = []
    for (W, A, B), g in zip(cases, groups):
        items.append(dict(W=dev(W), A=dev(A), B=dev(B), group=g, M=None))
    items = _with_filler(items)
    got = fq.qf_lora_merge_tensor_scale_nvfp4_grouped(items, 6).cpu().numpy()
    for g in range(5):
        members = [lora.merge(W, A, B) for (W, A, B), gg in zip(cases, groups) if gg == g]
        assert f32bits(got[g]) == f32bits(nvfp4.tensor_scale(members)), f"group {g}"
