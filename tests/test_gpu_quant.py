"""GPU parity: the HIP QDQ / pack / STE kernels against the CPU oracle, bit for bit.

Every comparison is exact: QDQ'd bf16 values, packed code bytes, block-scale
bytes, Q4_K blocks, tensor scales and STE outputs.  Inputs come from the
seeded workload generators (the 256x512 matrix with outliers, the 8B-layer
set, the Q4_K set) and from planted edge cases: ragged shapes spanning several
tiles, strided rows, in-place calls, signed zeros, subnormals, huge values and
a tied group whose tensor scale is tiny enough that 1/d overflows.
"""

import numpy as np
import pytest
import torch

import fp4_fake_quant_amd as fq
import workloads
from oracle import nvfp4, mxfp4, q4k, ste
from oracle import primitives as P
from tests import pins
from tests.gpu_util import dev, host, u8, f32bits, first_mismatch, sample_rows

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2024)


def _bits(x):
    return P.f32_to_bf16(np.asarray(x, np.float32))


# --------------------------------------------------------- oracle helpers --
def oracle_nvfp4(W, s_t):
    c, S = nvfp4.quantize(W, s_t)
    pc, ps = nvfp4.pack(c, S)
    return nvfp4.dequantize(c, S, s_t), pc, ps


def oracle_mxfp4(W):
    c, E = mxfp4.quantize(W)
    pc, ps = mxfp4.pack(c, E)
    return mxfp4.dequantize(c, E), pc, ps


def oracle_q4k(W):
    p = q4k.quantize(W)
    return q4k.dequantize(p), q4k.pack(p)


def assert_same(got, want, what):
    assert np.array_equal(got, want), f"{what}: {first_mismatch(got, want)}"


# -------------------------------------------------------- self-test ----
def test_conversion_instructions_conform():
    counts = fq.qf_selftest_conversions()
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8


# ------------------------------------------------- 256x512 workload ----
def test_nvfp4_single_matrix(single):
    W = single["W"]
    Wd = dev(W)
    s_ref = nvfp4.tensor_scale([W])
    d_scale = fq.qf_nvfp4_tensor_scale(Wd)
    assert f32bits(d_scale.cpu().numpy())[0] == f32bits(s_ref)
    y, codes, scales = fq.qf_qdq_pack_nvfp4(Wd, d_scale)
    y_ref, pc, ps = oracle_nvfp4(W, s_ref)
    assert_same(host(y), y_ref, "nvfp4 y")
    assert_same(u8(codes), pc, "nvfp4 codes")
    assert_same(u8(scales), ps, "nvfp4 scales")
    assert_same(host(fq.qf_qdq_nvfp4(Wd, d_scale)), y_ref, "nvfp4 qdq-only")
    c2, s2 = fq.qf_pack_nvfp4(Wd, d_scale)
    assert_same(u8(c2), pc, "nvfp4 pack-only codes")
    assert_same(u8(s2), ps, "nvfp4 pack-only scales")


def test_mxfp4_single_matrix(single):
    W = single["W"]
    Wd = dev(W)
    y, codes, scales = fq.qf_qdq_pack_mxfp4(Wd)
    y_ref, pc, ps = oracle_mxfp4(W)
    assert_same(host(y), y_ref, "mxfp4 y")
    assert_same(u8(codes), pc, "mxfp4 codes")
    assert_same(u8(scales), ps, "mxfp4 scales")
    assert_same(host(fq.qf_qdq_mxfp4(Wd)), y_ref, "mxfp4 qdq-only")
    c2, s2 = fq.qf_pack_mxfp4(Wd)
    assert_same(u8(c2), pc, "mxfp4 pack-only")
    assert_same(u8(s2), ps, "mxfp4 pack-only scales")


def test_q4k_single_matrix(single):
    W = single["W"]
    Wd = dev(W)
    y, blocks = fq.qf_qdq_pack_q4k(Wd)
    y_ref, b_ref = oracle_q4k(W)
    assert_same(host(y), y_ref, "q4k y")
    assert_same(u8(blocks), b_ref, "q4k blocks")
    assert_same(host(fq.qf_qdq_q4k(Wd)), y_ref, "q4k qdq-only")
    assert_same(u8(fq.qf_pack_q4k(Wd)), b_ref, "q4k pack-only")


def test_ste_single_matrix(single):
    G = single["G"]
    Gd = dev(G)
    out = fq.qf_ste_backward(Gd)
    assert_same(f32bits(out.cpu().numpy()), f32bits(ste.ste_backward(G)), "ste")
    acc = torch.randn(G.shape, device="cuda", dtype=torch.float32)
    acc_h = acc.cpu().numpy()
    fq.qf_ste_backward(Gd, acc, accumulate=True)
    assert_same(f32bits(acc.cpu().numpy()), f32bits(ste.ste_backward(G, acc_h, accumulate=True)), "ste accumulate")


# ---------------------------------------------------------- edge cases ----
def _special(rows, cols):
    x = RNG.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(RNG.integers(-20, 20, size=(rows, 1))).astype(np.float32)
    b = _bits(x)
    k = min(rows, 6)
    b[0 % rows, :] = 0
    if k > 1:
        b[1, :] = 0x8000
    if k > 2:
        b[2, :] = RNG.integers(1, 0x80, size=cols)            # subnormals
    if k > 3:
        b[3, :] = RNG.integers(0x8001, 0x8080, size=cols)
    if k > 4:
        b[4, ::7] = 0x8000                                      # scattered -0
    if k > 5:
        b[5, :] = RNG.integers(0x7E00, 0x7F7F, size=cols)       # huge
    return b


SHAPES = {
    "nvfp4": [(3, 48), (1, 16), (1000, 48), (7, 4096), (130, 160)],
    "mxfp4": [(5, 96), (1, 32), (999, 96), (7, 4096), (65, 224)],
    "q4k": [(3, 512), (1, 256), (513, 256), (7, 4096), (33, 768)],
}


@pytest.mark.parametrize("shape", SHAPES["nvfp4"])
def test_nvfp4_ragged_and_special(shape):
    W = _special(*shape) if shape[0] > 6 else _bits(RNG.standard_normal(shape) * 0.05)
    s_ref = nvfp4.tensor_scale([W])
    d_scale = fq.qf_nvfp4_tensor_scale(dev(W))
    assert f32bits(d_scale.cpu().numpy())[0] == f32bits(s_ref)
    y, c, s = fq.qf_qdq_pack_nvfp4(dev(W), d_scale)
    y_ref, pc, ps = oracle_nvfp4(W, s_ref)
    assert_same(host(y), y_ref, f"nvfp4 y {shape}")
    assert_same(u8(c), pc, f"nvfp4 codes {shape}")
    assert_same(u8(s), ps, f"nvfp4 scales {shape}")


@pytest.mark.parametrize("shape", SHAPES["mxfp4"])
def test_mxfp4_ragged_and_special(shape):
    W = _special(*shape) if shape[0] > 6 else _bits(RNG.standard_normal(shape) * 0.05)
    y, c, s = fq.qf_qdq_pack_mxfp4(dev(W))
    y_ref, pc, ps = oracle_mxfp4(W)
    assert_same(host(y), y_ref, f"mxfp4 y {shape}")
    assert_same(u8(c), pc, f"mxfp4 codes {shape}")
    assert_same(u8(s), ps, f"mxfp4 scales {shape}")


@pytest.mark.parametrize("shape", SHAPES["q4k"])
def test_q4k_ragged_and_special(shape):
    W = _special(*shape) if shape[0] > 6 else _bits(RNG.standard_normal(shape) * 0.05 + 0.01)
    if shape[0] > 6:
        W[5, :] = _bits(RNG.standard_normal(shape[1]) * 100)    # keep fp16 d finite: no huge row
    y, b = fq.qf_qdq_pack_q4k(dev(W))
    y_ref, b_ref = oracle_q4k(W)
    assert_same(host(y), y_ref, f"q4k y {shape}")
    assert_same(u8(b), b_ref, f"q4k blocks {shape}")


def test_nvfp4_tiny_group_scale_overflowing_reciprocal():
    """All values are bf16 subnormals: s_t is an fp32 subnormal and 1/d overflows."""
    W = RNG.integers(1, 0x80, size=(4, 64)).astype(np.uint16)
    W[1] |= 0x8000
    W[2, ::3] = 0
    W[3, ::5] = 0x8000
    s_ref = nvfp4.tensor_scale([W])
    d_scale = fq.qf_nvfp4_tensor_scale(dev(W))
    assert f32bits(d_scale.cpu().numpy())[0] == f32bits(s_ref)
    y, c, s = fq.qf_qdq_pack_nvfp4(dev(W), d_scale)
    y_ref, pc, ps = oracle_nvfp4(W, s_ref)
    assert_same(u8(c), pc, "codes")
    assert_same(u8(s), ps, "scales")
    assert_same(host(y), y_ref, "y")


def test_strided_rows_and_in_place():
    base = _bits(RNG.standard_normal((64, 1024)) * 0.03)
    Bd = dev(base)
    X = Bd[:, 256:768]                                       # ldx = 1024, cols = 512
    assert X.stride(0) == 1024
    W = base[:, 256:768]
    Yfull = torch.zeros((64, 640), dtype=torch.bfloat16, device="cuda")
    Y = Yfull[:, 64:576]                                     # ldy = 640
    fq.qf_qdq_mxfp4(X, Y)
    assert_same(host(Y), mxfp4.qdq(W), "mxfp4 strided")
    assert_same(host(Yfull[:, :64]), np.zeros((64, 64), np.uint16), "untouched left margin")
    fq.qf_qdq_q4k(X, Y)
    assert_same(host(Y), q4k.qdq(W), "q4k strided")
    d_scale = fq.qf_nvfp4_tensor_scale(X)
    s_ref = nvfp4.tensor_scale([W])
    assert f32bits(d_scale.cpu().numpy())[0] == f32bits(s_ref)
    fq.qf_qdq_nvfp4(X, d_scale, Y)
    assert_same(host(Y), nvfp4.qdq(W, s_ref), "nvfp4 strided")
    # in place
    Z = dev(W)
    fq.qf_qdq_nvfp4(Z, d_scale, Z)
    assert_same(host(Z), nvfp4.qdq(W, s_ref), "nvfp4 in place")


def test_nonfinite_flag():
    W = _bits(RNG.standard_normal((8, 64)))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.qf_nvfp4_tensor_scale(dev(W), d_nonfinite=flag)
    assert flag.item() == 0
    W[3, 17] = 0x7F80                                         # +inf
    fq.qf_nvfp4_tensor_scale(dev(W), d_nonfinite=flag)
    assert flag.item() == 1


def test_ste_ragged_lengths():
    for n in (1, 7, 8, 9, 8191, 8192 * 3 + 5):
        G = _bits(RNG.standard_normal(n))
        out = fq.qf_ste_backward(dev(G))
        assert_same(f32bits(out.cpu().numpy()), f32bits(ste.ste_backward(G)), f"ste n={n}")


# ------------------------------------------------------ tying / grouping ----
def test_nvfp4_pointer_array_tensor_scale():
    """qf_nvfp4_tensor_scale over a host array of pointers (Q, K, V as separate contiguous
    tensors, one tied group) gives the fused matrix's scale; also with a single tensor, an
    empty member, and a member whose length is a multiple of 16 but not of a row."""
    q = _bits(RNG.standard_normal((512, 256)) * 0.02)
    k = _bits(RNG.standard_normal((128, 256)) * 0.05)
    v = _bits(RNG.standard_normal((128, 256)) * 0.01)
    ts = [dev(t) for t in (q, k, v)]
    got = fq.qf_nvfp4_tensor_scale(ts)
    assert f32bits(got.cpu().numpy()[0]) == f32bits(nvfp4.tensor_scale([np.concatenate([q, k, v])]))
    assert f32bits(fq.qf_nvfp4_tensor_scale(ts[1]).cpu().numpy()[0]) == f32bits(nvfp4.tensor_scale([k]))
    flat = dev(q).reshape(-1)[: 16 * 1001]
    empty = dev(q).reshape(-1)[:0]
    got = fq.qf_nvfp4_tensor_scale([flat, empty, ts[2]])
    want = nvfp4.tensor_scale([q.reshape(-1)[: 16 * 1001].reshape(1001, 16), v])
    assert f32bits(got.cpu().numpy()[0]) == f32bits(want)


def test_nvfp4_tied_qkv_equals_fused():
    q = _bits(RNG.standard_normal((512, 256)) * 0.02)
    k = _bits(RNG.standard_normal((128, 256)) * 0.05)
    v = _bits(RNG.standard_normal((128, 256)) * 0.01)
    o = _bits(RNG.standard_normal((256, 512)) * 0.03)
    ts = [dev(t) for t in (q, k, v, o)]
    scales = fq.qf_nvfp4_tensor_scale_grouped(
        [dict(x=ts[0], group=0), dict(x=ts[1], group=0), dict(x=ts[2], group=0), dict(x=ts[3], group=1)], 2)
    s_qkv = nvfp4.tensor_scale([q, k, v])
    s_o = nvfp4.tensor_scale([o])
    assert np.array_equal(f32bits(scales.cpu().numpy()), f32bits([s_qkv, s_o]))
    outs = []
    items = []
    for t, g, h in zip(ts, (0, 0, 0, 1), (q, k, v, o)):
        y = torch.empty_like(t)
        c = torch.empty((h.shape[0], h.shape[1] // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((h.shape[0], h.shape[1] // 16), dtype=torch.uint8, device="cuda")
        outs.append((y, c, s))
        items.append(dict(x=t, y=y, codes=c, scales=s, group=g))
    items[3]["y"] = None                                       # pack-only for O: a second launch
    fq.qf_qdq_pack_nvfp4_grouped(items, scales)
    fused = np.concatenate([q, k, v])
    y_ref, pc, ps = oracle_nvfp4(fused, s_qkv)
    assert_same(np.concatenate([host(outs[i][0]) for i in range(3)]), y_ref, "tied y")
    assert_same(np.concatenate([u8(outs[i][1]) for i in range(3)]), pc, "tied codes")
    assert_same(np.concatenate([u8(outs[i][2]) for i in range(3)]), ps, "tied scales")
    _, pco, pso = oracle_nvfp4(o, s_o)
    assert_same(u8(outs[3][1]), pco, "O codes")
    assert_same(u8(outs[3][2]), pso, "O scales")


# ---------------------------------------------- full-size workloads ----
def test_dense_layer_8b_nvfp4_full_size():
    """The 8B-layer set at full size: grouped tensor scales and grouped QDQ+pack in the
    launch configuration the benchmark times; the oracle checks every tensor scale
    exactly and 64 sampled rows (plus first and last) of every output per matrix."""
    layer = workloads.dense_layer_8b(with_grad=True)
    names = list(layer)
    Ws = {n: dev(layer[n][0]) for n in names}
    items = [dict(x=Ws[n], group=i) for i, n in enumerate(names)]
    scales = fq.qf_nvfp4_tensor_scale_grouped(items, len(names))
    outs = {}
    qitems = []
    for i, n in enumerate(names):
        r, c = layer[n][0].shape
        outs[n] = (torch.empty_like(Ws[n]), torch.empty((r, c // 2), dtype=torch.uint8, device="cuda"),
                   torch.empty((r, c // 16), dtype=torch.uint8, device="cuda"))
        qitems.append(dict(x=Ws[n], y=outs[n][0], codes=outs[n][1], scales=outs[n][2], group=i))
    fq.qf_qdq_pack_nvfp4_grouped(qitems, scales)
    sc = scales.cpu().numpy()
    for i, n in enumerate(names):
        W, G = layer[n]
        s_ref = nvfp4.tensor_scale([W])
        assert f32bits(sc[i]) == f32bits(s_ref), n
        rows = sample_rows(W.shape[0], 64, seed=i)
        y_ref, pc, ps = oracle_nvfp4(W[rows], s_ref)
        assert_same(host(outs[n][0])[rows], y_ref, f"{n} y")
        assert_same(u8(outs[n][1])[rows], pc, f"{n} codes")
        assert_same(u8(outs[n][2])[rows], ps, f"{n} scales")
        g = fq.qf_ste_backward(dev(G))
        gh = g.cpu().numpy()
        assert_same(f32bits(gh[rows]), f32bits(ste.ste_backward(G[rows])), f"{n} ste")
        del g


def test_q4k_set_full_size_sampled():
    names = ["single", "qkv", "o", "vocab"]
    tens = workloads.q4k_set(names=names)
    items, outs = [], {}
    for n in names:
        W = tens[n]
        r, c = W.shape
        Wd = dev(W)
        outs[n] = (Wd, torch.empty_like(Wd), torch.empty((r, c // 256, 144), dtype=torch.uint8, device="cuda"))
        items.append(dict(x=Wd, y=outs[n][1], codes=outs[n][2]))
    fq.qf_qdq_pack_q4k_grouped(items)
    for i, n in enumerate(names):
        W = tens[n]
        rows = sample_rows(W.shape[0], 48, seed=10 + i)
        y_ref, b_ref = oracle_q4k(W[rows])
        assert_same(host(outs[n][1])[rows], y_ref, f"{n} y")
        assert_same(u8(outs[n][2])[rows], b_ref, f"{n} blocks")


def test_q4k_set_all_six_one_launch():
    """The benchmark's Q4_K launch: all six tensors of the Q4_K set (256 x 512, QKV,
    gate/up, down, O and the 151936 x 4096 vocabulary) in one grouped call, drawn on the
    device with the same recipe; sampled rows of every tensor, copied to the host, against
    the oracle bit for bit (y and 144-byte blocks)."""
    tens = workloads.q4k_set_device()
    names = list(tens)
    assert len(names) == 6
    items, outs = [], {}
    for n in names:
        Wd = tens[n]
        r, c = Wd.shape
        outs[n] = (torch.empty_like(Wd), torch.empty((r, c // 256, 144), dtype=torch.uint8, device="cuda"))
        items.append(dict(x=Wd, y=outs[n][0], codes=outs[n][1]))
    fq.qf_qdq_pack_q4k_grouped(items)
    torch.cuda.synchronize()
    for i, n in enumerate(names):
        rows = sample_rows(tens[n].shape[0], 24, seed=40 + i)
        ri = torch.from_numpy(rows).cuda()
        W = host(tens[n][ri])
        y_ref, b_ref = oracle_q4k(W)
        assert_same(host(outs[n][0][ri]), y_ref, f"{n} y")
        assert_same(u8(outs[n][1][ri]), b_ref, f"{n} blocks")


def test_mxfp4_gemm_operands_full_size_sampled():
    g = workloads.w4a4_gemm()
    for name in ("X", "W"):
        A = g[name]
        y, c, s = fq.qf_qdq_pack_mxfp4(dev(A))
        rows = sample_rows(A.shape[0], 64, seed=3)
        y_ref, pc, ps = oracle_mxfp4(A[rows])
        assert_same(host(y)[rows], y_ref, f"{name} y")
        assert_same(u8(c)[rows], pc, f"{name} codes")
        assert_same(u8(s)[rows], ps, f"{name} scales")
        del y, c, s


# ------------------------------------------------- MXFP4 noclip exponent rule ----
def _mx_rule_items(x_bits):
    xd = dev(x_bits)
    rows, cols = x_bits.shape
    it = dict(x=xd, y=torch.empty_like(xd),
              codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
              scales=torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda"))
    return it


@pytest.mark.parametrize("which", ["single", "planted", "ragged"])
def test_mxfp4_noclip_rule(single, which):
    """QF_MX_RULE_NOCLIP against the oracle bit for bit (y, codes, E8M0 bytes); the floor
    rule through the same entry point equals qf_qdq_pack_mxfp4."""
    if which == "single":
        x = single["W"]
    elif which == "planted":
        x = pins.planted_mx_blocks()
    else:
        x = workloads.to_bf16_bits(np.random.default_rng(3).standard_t(3, size=(37, 96)).astype(np.float32))
    it = _mx_rule_items(x)
    fq.qf_qdq_pack_mxfp4_rule([it], fq.QF_MX_RULE_NOCLIP)
    c, E = mxfp4.quantize(x, rule="noclip")
    pc, ps = mxfp4.pack(c, E)
    assert_same(host(it["y"]), mxfp4.dequantize(c, E), "noclip y")
    assert_same(u8(it["codes"]), pc, "noclip codes")
    assert_same(u8(it["scales"]), ps, "noclip E")
    assert_same(host(fq.qf_dequant_mxfp4(it["codes"], it["scales"])), host(it["y"]), "noclip dequant")
    fq.qf_qdq_pack_mxfp4_rule([it], fq.QF_MX_RULE_FLOOR)
    y, c2, s2 = fq.qf_qdq_pack_mxfp4(it["x"])
    assert_same(host(it["y"]), host(y), "floor rule y")
    assert_same(u8(it["scales"]), u8(s2), "floor rule E")


# --------------------------------------------------- Q4_K mse scale rule ----
def _q4k_rule_items(x_bits):
    xd = dev(x_bits)
    rows, cols = x_bits.shape
    return dict(x=xd, y=torch.empty_like(xd),
                codes=torch.empty((rows, cols // 256, 144), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("which", ["single", "asymmetric", "ragged", "on_grid"])
def test_q4k_mse_rule(single, which):
    """QF_Q4K_RULE_MSE against the oracle bit for bit (y and the 144-byte blocks), dequant of
    the blocks equal to y, and the min/max rule through the same entry point equal to
    qf_qdq_pack_q4k."""
    rng = np.random.default_rng(11)
    if which == "single":
        x = single["W"]
    elif which == "asymmetric":                      # the Q4_K set's recipe: mean 0.001, row offsets
        x = workloads.to_bf16_bits((np.float32(0.001) + np.float32(0.02) * rng.standard_normal((64, 1024))
                                    + rng.uniform(-0.01, 0.01, (64, 1)).astype(np.float32)).astype(np.float32))
    elif which == "ragged":
        x = workloads.to_bf16_bits(rng.standard_t(3, size=(37, 768)).astype(np.float32))
    else:                                            # every sub-block on its own min/max grid
        lvl = np.stack([rng.permutation(np.arange(16).repeat(2)) for _ in range(16 * 16)]).reshape(16, 512)
        x = workloads.to_bf16_bits((np.float32(-0.5) + np.float32(0.0625) * lvl).astype(np.float32))
    it = _q4k_rule_items(x)
    fq.qf_qdq_pack_q4k_rule([it], fq.QF_Q4K_RULE_MSE)
    p = q4k.quantize(x, "mse")
    assert_same(host(it["y"]), q4k.dequantize(p), f"mse y ({which})")
    assert_same(u8(it["codes"]), q4k.pack(p), f"mse blocks ({which})")
    assert_same(host(fq.qf_dequant_q4k(it["codes"], *x.shape)), host(it["y"]), f"mse dequant ({which})")
    fq.qf_qdq_pack_q4k_rule([it], fq.QF_Q4K_RULE_MINMAX)
    y, b = fq.qf_qdq_pack_q4k(it["x"])
    assert_same(host(it["y"]), host(y), "minmax rule y")
    assert_same(u8(it["codes"]), u8(b), "minmax rule blocks")


def test_q4k_mse_rule_full_size_sampled():
    """The Q4_K set's gate/up and vocabulary matrices at full size under the mse rule, one
    grouped launch; the oracle checks sampled rows bit for bit."""
    names = ["gate_up", "vocab"]
    tens = workloads.q4k_set(names=names)
    items = [_q4k_rule_items(tens[n]) for n in names]
    fq.qf_qdq_pack_q4k_rule(items, fq.QF_Q4K_RULE_MSE)
    for n, it in zip(names, items):
        x = tens[n]
        rows = sample_rows(x.shape[0], 24, seed=len(n))
        ri = torch.from_numpy(rows).cuda()
        p = q4k.quantize(x[rows], "mse")
        assert_same(host(it["y"][ri]), q4k.dequantize(p), f"{n} mse y")
        assert_same(u8(it["codes"][ri]), q4k.pack(p), f"{n} mse blocks")
    del items
    torch.cuda.empty_cache()
