"""The C-ABI library loads and exports every entry point include/qf.h declares.

Host-only checks (no GPU needed): symbol table, helper results, and argument
validation, which returns before anything is enqueued.
"""

import ctypes
import os
import re

import pytest

from fp4_fake_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qf_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    # the Python signatures cover exactly the declared entry points
    assert sorted(_lib.SIGNATURES) == names


def test_helpers_host_only():
    L = _lib.lib()
    assert L.qf_version() >> 8 == 1
    assert L.qf_status_str(0) == b"ok"
    assert L.qf_packed_bytes(0, 256, 512) == 73_728          # + 4 bytes of fp32 tensor scale = 73,732
    assert L.qf_packed_bytes(1, 256, 512) == 69_632
    assert L.qf_packed_bytes(2, 256, 512) == 73_728
    assert L.qf_packed_bytes(0, 256, 24) == 0                # not a block multiple
    assert L.qf_packed_bytes(7, 1, 16) == 0


def _addr(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("case", ["null_x", "bad_cols", "ld_small", "misaligned", "neg_rows"])
def test_argument_validation_returns_before_launch(case):
    """Invalid arguments come back as status codes; fake non-null addresses are never touched."""
    L = _lib.lib()
    good = 0x10000000
    x, y = good, good + 0x100000
    rows, cols, ldx, ldy = 4, 64, 64, 64
    if case == "null_x":
        x = 0
    if case == "bad_cols":
        cols = ldx = ldy = 40
    if case == "ld_small":
        ldx = 32
    if case == "misaligned":
        x = good + 2
    if case == "neg_rows":
        rows = -1
    st = L.qf_qdq_mxfp4(_addr(x) if x else None, rows, cols, ldx, _addr(y), ldy, None)
    expect = {"null_x": 1, "bad_cols": 2, "ld_small": 2, "misaligned": 3, "neg_rows": 2}[case]
    assert st == expect


def test_validation_of_other_entry_points():
    L = _lib.lib()
    p = _addr(0x10000000)
    q = _addr(0x10100000)
    assert L.qf_qdq_nvfp4(p, 4, 64, 64, None, q, 64, None) == 1            # missing tensor scale
    assert L.qf_qdq_q4k(p, 4, 128, 128, q, 128, None) == 2                 # 128 is not a 256 multiple
    assert L.qf_pack_mxfp4(p, 4, 64, 64, q, None, None) == 1               # missing scales
    assert L.qf_pack_q4k(p, 4, 256, 256, _addr(0x10100004), None) == 3     # blocks must be 16-byte aligned
    assert L.qf_ste_backward(p, _addr(0x10100004), 100, 0, None) == 3
    assert L.qf_ste_backward(None, q, 100, 0, None) == 1
    assert L.qf_ste_backward(p, q, 0, 0, None) == 0                        # empty: no-op
    assert L.qf_qdq_mxfp4(p, 0, 64, 64, q, 64, None) == 0                  # empty: no-op
    assert L.qf_selftest_conversions(None, None) == 1
    # tensor scale: workspace must be given and large enough
    d = (_lib.TensorDesc * 1)()
    d[0].x, d[0].rows, d[0].cols, d[0].ldx, d[0].group = 0x10000000, 1024, 4096, 4096, 0
    need = L.qf_nvfp4_tensor_scale_workspace(ctypes.byref(d), 1)
    assert need > 0 and need % 4 == 0
    assert L.qf_nvfp4_tensor_scale_grouped(ctypes.byref(d), 1, 1, q, None, None, 0, None) == 4
    assert L.qf_nvfp4_tensor_scale_grouped(ctypes.byref(d), 1, 1, q, None, q, need - 4, None) == 4
    d[0].group = 3
    assert L.qf_nvfp4_tensor_scale_grouped(ctypes.byref(d), 1, 2, q, None, q, need, None) == 7
    assert L.qf_qdq_pack_mxfp4_grouped(ctypes.byref(d), 17, None) == 7      # too many tensors


def test_lora_validation():
    """LoRA calls check rank, shape, group and workspace before launching."""
    L = _lib.lib()
    q = _addr(0x10100000)
    d = (_lib.LoraDesc * 2)()
    for i in range(2):
        d[i].W, d[i].rows, d[i].cols, d[i].ldw = 0x10000000, 100, 1056, 1056
        d[i].A, d[i].B, d[i].r, d[i].group = 0x10200000, 0x10300000, 16, i
        d[i].M, d[i].G, d[i].dA, d[i].dB = 0x10400000, 0x10500000, 0x10600000, 0x10700000
    need = L.qf_lora_workspace(ctypes.byref(d), 2)
    assert need > 0 and need % 4 == 0
    # a launch this small shrinks its merge units to the minimum of 8 rows:
    # merge partials ceil(ceil(100/8) * 3 slabs / 4) = 10 workgroups per matrix x 2 groups;
    # gradient partials: dA one 256-row block x 16 x 1056, dB 3 slabs x 100 rows x 16, per matrix
    assert need == 4 * max(20 * 2, 2 * (16 * 1056 + 3 * 100 * 16))
    assert L.qf_lora_merge_tensor_scale_nvfp4_grouped(ctypes.byref(d), 2, 2, q, None, q, need - 4, None) == 4
    assert L.qf_lora_merge_tensor_scale_nvfp4_grouped(ctypes.byref(d), 2, 1, q, None, q, need, None) == 7   # group 1 >= 1
    assert L.qf_lora_adapter_grads_grouped(ctypes.byref(d), 2, 0, None, 0, None) == 4
    d[1].r = 17
    assert L.qf_lora_workspace(ctypes.byref(d), 2) == 0
    assert L.qf_lora_merge_tensor_scale_nvfp4_grouped(ctypes.byref(d), 2, 2, q, None, q, need, None) == 7
    d[1].r = 16
    d[1].ldw = 1 << 24                                              # row stride too large
    assert L.qf_lora_adapter_grads_grouped(ctypes.byref(d), 2, 0, q, need, None) == 2
    d[1].cols = d[1].ldw = 1048                                     # not a multiple of 32
    assert L.qf_lora_adapter_grads_grouped(ctypes.byref(d), 2, 0, q, need, None) == 2
    d[1].cols = d[1].ldw = 1056
    d[1].B = 0x10300002                                             # B must be 4-byte aligned
    assert L.qf_lora_adapter_grads_grouped(ctypes.byref(d), 2, 0, q, need, None) == 3
    d[1].B = 0x10300000
    d[0].W = 0                                                      # W is needed (M may be NULL)
    assert L.qf_lora_merge_tensor_scale_nvfp4_grouped(ctypes.byref(d), 2, 2, q, None, q, need, None) == 1
    d[0].W = 0x10000000
    # QDQ pass: an output is required; without M, W / A / B are read and checked
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, q, None) == 1            # no y and no codes
    d[0].y, d[1].y = 0x10800000, 0x10900000
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, None, None) == 1         # no tensor scales
    d[0].M = 0
    d[0].W = 0x10000008                                             # W must be 16-byte aligned
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, q, None) == 3
    d[0].W = 0x10000000
    d[0].A = 0
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, q, None) == 1
    d[0].A = 0x10200000
    d[0].y = 0x10800008                                             # y must be 16-byte aligned
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, q, None) == 3
    d[0].group = -1
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 2, q, None) == 7
    assert L.qf_lora_merge_qdq_pack_nvfp4_grouped(ctypes.byref(d), 17, q, None) == 7
    d[0].rows = d[1].rows = 0                                       # empty: nothing to do
    assert L.qf_lora_adapter_grads_grouped(ctypes.byref(d), 2, 0, q, 4, None) == 0


def test_lora_gradient_unit_rows():
    """Gradient workgroups take 512 rows when that still gives 256 of them, else 256
    (the workspace holds one dA partial per unit): 16 matrices of 600 x 4096 take 2 units
    of 512 rows each, 2 such matrices take 3 of 256."""
    L = _lib.lib()
    d = (_lib.LoraDesc * 16)()
    for i in range(16):
        d[i].W, d[i].rows, d[i].cols, d[i].ldw = 0x10000000, 600, 4096, 4096
        d[i].A, d[i].B, d[i].r, d[i].group = 0x10200000, 0x10300000, 16, i
    dB = 8 * 600 * 16                                              # 8 slabs per matrix
    assert L.qf_lora_workspace(ctypes.byref(d), 16) == 4 * 16 * (2 * 16 * 4096 + dB)
    assert L.qf_lora_workspace(ctypes.byref(d), 2) == 4 * 2 * (3 * 16 * 4096 + dB)


def test_mxfp4_rule_validation():
    L = _lib.lib()
    d = (_lib.TensorDesc * 1)()
    d[0].x, d[0].rows, d[0].cols, d[0].ldx = 0x10000000, 4, 64, 64
    d[0].y, d[0].ldy = 0x10400000, 64
    assert L.qf_qdq_pack_mxfp4_rule(ctypes.byref(d), 1, 2, None) == 7           # unknown rule
    assert L.qf_qdq_pack_mxfp4_rule(ctypes.byref(d), 1, -1, None) == 7
    d[0].cols = d[0].ldx = d[0].ldy = 48                                         # not a multiple of 32
    assert L.qf_qdq_pack_mxfp4_rule(ctypes.byref(d), 1, 1, None) == 2


def test_q4k_rule_validation():
    L = _lib.lib()
    d = (_lib.TensorDesc * 1)()
    d[0].x, d[0].rows, d[0].cols, d[0].ldx = 0x10000000, 4, 512, 512
    d[0].y, d[0].ldy = 0x10400000, 512
    assert L.qf_qdq_pack_q4k_rule(ctypes.byref(d), 1, 2, None) == 7             # unknown rule
    assert L.qf_qdq_pack_q4k_rule(ctypes.byref(d), 1, -1, None) == 7
    d[0].cols = d[0].ldx = d[0].ldy = 384                                        # not a multiple of 256
    assert L.qf_qdq_pack_q4k_rule(ctypes.byref(d), 1, 1, None) == 2


def test_transpose_and_backward_validation():
    L = _lib.lib()
    x, y, w, d = _addr(0x10000000), _addr(0x10400000), _addr(0x10800000), _addr(0x10c00000)
    assert L.qf_transpose_bf16(x, 12, 64, 64, y, 16, 0, None) == 2             # rows not a multiple of 8
    assert L.qf_transpose_bf16(x, 16, 48, 48, y, 16, 1, None) == 2             # QDQ needs 32-blocks
    assert L.qf_transpose_bf16(x, 16, 48, 48, y, 8, 0, None) == 2              # ldy < rows
    assert L.qf_transpose_bf16(_addr(0x10000008), 16, 48, 48, y, 16, 0, None) == 3
    assert L.qf_transpose_bf16(x, 0, 48, 48, y, 16, 0, None) == 0              # empty: no-op
    assert L.qf_transpose_bf16(x, 16, 64, 64, y, 16, 3, None) == 7             # unknown QDQ mode
    assert L.qf_transpose_bf16(x, 16, 64, 64, y, 16, -1, None) == 7
    need = L.qf_linear_backward_workspace(128, 64, 96)
    assert need == 96 * 64 * 2 + 64 * 128 * 2 + 96 * 128 * 2
    args = (x, 96, w, 96, d, 64, y, 96, _addr(0x11000000), 96)
    assert L.qf_linear_backward_mxfp4(*args, 100, 64, 96, 3, _addr(0x12000000), need, None) == 2   # M % 64
    assert L.qf_linear_backward_mxfp4(*args, 128, 64, 80, 3, _addr(0x12000000), need, None) == 2   # K % 32
    assert L.qf_linear_backward_mxfp4(*args, 128, 64, 96, 4, _addr(0x12000000), need, None) == 7   # flags
    assert L.qf_linear_backward_mxfp4(*args, 128, 64, 96, 8, _addr(0x12000000), need, None) == 7   # noclip alone
    assert L.qf_linear_backward_mxfp4(*args, 128, 64, 96, 3, _addr(0x12000000), need - 2, None) == 4
    assert L.qf_linear_backward_mxfp4(*args, 128, 64, 96, 3, _addr(0x12000010), need, None) == 3   # ws alignment
    assert L.qf_linear_backward_mxfp4(x, 96, None, 96, d, 64, y, 96, None, 0, 128, 64, 96, 3,
                                      _addr(0x12000000), need, None) == 1                          # dX needs W


def test_linear_forward_validation():
    """The two-pass forward checks every argument before its first launch."""
    L = _lib.lib()
    x, w, y, xq, wq, f = (_addr(a) for a in (0x10000000, 0x10400000, 0x10800000, 0x10c00000, 0x11000000, 0x11400000))
    mx = lambda *a: L.qf_linear_forward_mxfp4(*a, None)
    assert mx(x, 128, w, 128, y, 64, 64, 64, 96, 3, xq, 128, wq, 128) == 2            # K % 64
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 16, xq, 128, wq, 128) == 7          # unknown flag
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 8, xq, 128, wq, 128) == 7           # noclip with no operand
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 3, None, 128, wq, 128) == 1         # Xq needed
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 3, xq, 120, wq, 128) == 2           # ldxq < K
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 3, _addr(0x10c00008), 128, wq, 128) == 3
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 3, xq, 132, wq, 128) == 3           # ldxq % 8
    assert mx(x, 128, w, 128, y, 64, 64, 64, 128, 3, xq, 1 << 22, wq, 128) == 2       # ldxq >= 2^22
    assert mx(x, 128, w, 128, y, 64, 0, 64, 128, 3, None, 0, None, 0) == 0            # empty: no-op
    nv = lambda *a: L.qf_linear_forward_nvfp4(*a, None)
    assert nv(x, 128, w, 128, y, 64, 64, 64, 128, 0, f, f, xq, 128, wq, 128) == 7     # flags 0
    assert nv(x, 128, w, 128, y, 64, 64, 64, 128, 3, None, f, xq, 128, wq, 128) == 1  # scale of X
    assert nv(x, 128, w, 128, y, 64, 64, 64, 128, 3, _addr(0x11400002), f, xq, 128, wq, 128) == 3


def test_ste_clipped_validation():
    L = _lib.lib()
    g, x, o, f = _addr(0x10000000), _addr(0x10400000), _addr(0x10800000), _addr(0x10c00000)
    assert L.qf_ste_backward_clipped_mxfp4(g, x, 4, 48, 48, 0, o, 0, None) == 2        # cols % 32
    assert L.qf_ste_backward_clipped_nvfp4(g, x, 4, 24, 24, f, o, 0, None) == 2        # cols % 16
    assert L.qf_ste_backward_clipped_mxfp4(g, x, 4, 64, 64, 5, o, 0, None) == 7        # rule
    assert L.qf_ste_backward_clipped_nvfp4(g, x, 4, 32, 32, None, o, 0, None) == 1     # tensor scale
    assert L.qf_ste_backward_clipped_mxfp4(g, x, 4, 64, 32, 0, o, 0, None) == 2        # ldx < cols
    assert L.qf_ste_backward_clipped_mxfp4(g, _addr(0x10400008), 4, 64, 64, 0, o, 0, None) == 3
    assert L.qf_ste_backward_clipped_mxfp4(g, x, 4, 64, 68, 0, o, 0, None) == 3        # ldx % 8
    assert L.qf_ste_backward_clipped_nvfp4(g, x, 4, 32, 32, _addr(0x10c00002), o, 0, None) == 3
    assert L.qf_ste_backward_clipped_mxfp4(g, x, 0, 64, 64, 0, o, 0, None) == 0        # empty: no-op


def test_dequant_validation():
    """Dequant calls check shape, pointers and alignment before launching."""
    L = _lib.lib()
    c, s, y, f = _addr(0x10000000), _addr(0x10400000), _addr(0x10800000), _addr(0x10c00000)
    assert L.qf_dequant_nvfp4(c, s, 4, 24, f, y, 24, None) == 2                 # cols not a multiple of 16
    assert L.qf_dequant_mxfp4(c, s, 4, 48, y, 48, None) == 2                    # ... of 32
    assert L.qf_dequant_q4k(c, 4, 384, y, 384, None) == 2                       # ... of 256
    assert L.qf_dequant_nvfp4(c, s, 4, 32, None, y, 32, None) == 1              # NVFP4 needs the tensor scale
    assert L.qf_dequant_mxfp4(c, None, 4, 64, y, 64, None) == 1
    assert L.qf_dequant_nvfp4(c, s, 4, 32, f, y, 16, None) == 2                 # ldy < cols
    assert L.qf_dequant_mxfp4(c, s, 4, 64, _addr(0x10800008), 64, None) == 3    # y 16-byte aligned
    assert L.qf_dequant_mxfp4(c, s, 4, 64, y, 68, None) == 3                    # ldy a multiple of 8
    assert L.qf_dequant_q4k(_addr(0x10000004), 4, 256, y, 256, None) == 3       # blocks 16-byte aligned
    assert L.qf_dequant_q4k(c, 0, 256, y, 256, None) == 0                       # empty: no-op


def test_gemm_validation():
    """GEMM entry points check flags, K and alignment before launching."""
    L = _lib.lib()
    p, q, y = _addr(0x10000000), _addr(0x10400000), _addr(0x10800000)
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 4, None) == 7        # FP4 cores need both QDQ flags
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 5, None) == 7
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 8, None) == 7        # unknown flag
    assert L.qf_gemm_mxfp4(p, 96, q, 96, y, 64, 64, 64, 96, 3, None) == 2        # K not a multiple of 64
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 0, 64, 64, 7, None) == 0         # empty: no-op
    assert L.qf_gemm_mxfp4(p, 1 << 22, q, 64, y, 64, 64, 64, 64, 3, None) == 2   # a tile's offsets reach 2^31
    assert L.qf_gemm_mxfp4(p, 64, q, 1 << 22, y, 64, 64, 64, 64, 3, None) == 2
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 8, None) == 7        # noclip needs a QDQ flag
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 15, None) == 7       # noclip is BF16-core only
    assert L.qf_gemm_mxfp4(p, 64, q, 64, y, 64, 64, 64, 64, 16, None) == 7       # unknown flag
    s = _addr(0x10c00000)
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 64, 64, 0, s, s, None) == 7   # no operand quantized
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 64, 64, 7, s, s, None) == 7   # no FP4-core form
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 64, 64, 3, None, s, None) == 1
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 64, 64, 3, s, None, None) == 1
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 64, 64, 2, _addr(0x10c00002), s, None) == 3   # unused, but misaligned
    assert L.qf_gemm_nvfp4(p, 96, q, 96, y, 64, 64, 64, 96, 3, s, s, None) == 2   # K not a multiple of 64
    assert L.qf_gemm_nvfp4(p, 64, q, 64, y, 64, 64, 0, 64, 3, s, s, None) == 0    # empty: no-op
    xs, ws = _addr(0x10C00000), _addr(0x10E00000)
    assert L.qf_gemm_mxfp4_packed(p, xs, q, ws, y, 64, 64, 64, 64, None) == 2    # K not a multiple of 128
    assert L.qf_gemm_mxfp4_packed(p, _addr(0x10C00002), q, ws, y, 64, 64, 64, 128, None) == 3   # exponents 4-byte aligned
    assert L.qf_gemm_mxfp4_packed(None, xs, q, ws, y, 64, 64, 64, 128, None) == 1
    assert L.qf_gemm_mxfp4_packed(p, xs, q, ws, y, 32, 64, 64, 128, None) == 2   # ldy < N
    assert L.qf_gemm_mxfp4_packed(p, xs, q, ws, y, 64, 64, 0, 128, None) == 0    # empty: no-op
    assert L.qf_gemm_mxfp4_packed_w(p, 96, q, ws, y, 64, 64, 64, 96, None) == 2  # K not a multiple of 64
    assert L.qf_gemm_mxfp4_packed_w(p, 64, _addr(0x10400008), ws, y, 64, 64, 64, 64, None) == 3  # codes 16-byte aligned
    assert L.qf_gemm_mxfp4_packed_w(p, 64, q, None, y, 64, 64, 64, 64, None) == 1


# the calls of the boundary as the survey's contract lists them
SURVEY_BOUNDARY = [
    "qf_nvfp4_tensor_scale", "qf_qdq_nvfp4", "qf_qdq_mxfp4", "qf_qdq_q4k",
    "qf_pack_nvfp4", "qf_pack_mxfp4", "qf_pack_q4k",
    "qf_qdq_pack_nvfp4", "qf_qdq_pack_mxfp4", "qf_qdq_pack_q4k",
    "qf_nvfp4_tensor_scale_grouped", "qf_qdq_pack_nvfp4_grouped", "qf_qdq_pack_mxfp4_grouped",
    "qf_qdq_pack_q4k_grouped", "qf_ste_backward", "qf_gemm_mxfp4",
    "qf_lora_merge_tensor_scale_nvfp4", "qf_lora_merge_qdq_pack_nvfp4", "qf_lora_adapter_grads",
    "qf_packed_bytes", "qf_workspace_size", "qf_status_str", "qf_last_hip_error", "qf_version",
]


def test_survey_boundary_names_are_exported():
    L = _lib.lib()
    declared = declared_functions()
    for n in SURVEY_BOUNDARY:
        assert n in declared and hasattr(L, n), n


def test_pointer_array_tensor_scale_validation():
    """qf_nvfp4_tensor_scale over a host array of device pointers (one tied group)."""
    L = _lib.lib()
    q = _addr(0x10100000)
    ptrs = (ctypes.c_void_p * 3)(0x10000000, 0x10200000, 0x10400000)
    numel = (ctypes.c_int64 * 3)(6144 * 4096 // 3, 6144 * 4096 // 6, 6144 * 4096 // 6)
    need = L.qf_workspace_size(0, 1, numel[0], 3)
    assert need == 4 * 2048 * 64                                   # the persistent grid, 64 groups
    assert L.qf_nvfp4_tensor_scale(ptrs, numel, 3, q, None, None, 0, None) == 4
    assert L.qf_nvfp4_tensor_scale(ptrs, numel, 17, q, None, q, need, None) == 7
    assert L.qf_nvfp4_tensor_scale(ptrs, numel, 3, None, None, q, need, None) == 1
    assert L.qf_nvfp4_tensor_scale(None, numel, 3, q, None, q, need, None) == 1
    bad = (ctypes.c_int64 * 3)(4096, 4100, 16)                    # 4100 is not a multiple of 16
    assert L.qf_nvfp4_tensor_scale(ptrs, bad, 3, q, None, q, need, None) == 2
    odd = (ctypes.c_void_p * 3)(0x10000000, 0x10200008, 0x10400000)
    assert L.qf_nvfp4_tensor_scale(odd, numel, 3, q, None, q, need, None) == 3


def test_single_matrix_lora_validation():
    L = _lib.lib()
    W, A, B, G = (_addr(0x10000000 + 0x1000000 * i) for i in range(4))
    q = _addr(0x14000000)
    need = L.qf_workspace_size(1, 3072, 3072, 1)
    assert L.qf_lora_merge_tensor_scale_nvfp4(W, A, B, 3072, 3072, 16, q, q, need - 4, None) == 4
    assert L.qf_lora_merge_tensor_scale_nvfp4(W, A, B, 3072, 3072, 17, q, q, need, None) == 7   # rank
    assert L.qf_lora_merge_tensor_scale_nvfp4(W, A, B, 3072, 3000, 16, q, q, need, None) == 2   # cols % 32
    assert L.qf_lora_merge_tensor_scale_nvfp4(None, A, B, 3072, 3072, 16, q, q, need, None) == 1
    assert L.qf_lora_merge_qdq_pack_nvfp4(W, A, B, 3072, 3072, 16, q, None, None, None, None) == 1   # no output
    assert L.qf_lora_merge_qdq_pack_nvfp4(W, A, B, 3072, 3072, 16, None, q, None, None, None) == 1   # no scale
    assert L.qf_lora_merge_qdq_pack_nvfp4(W, A, B, 3072, 3072, 16, q, _addr(0x14000008), None, None, None) == 3
    assert L.qf_lora_adapter_grads(G, A, B, 3072, 3072, 16, q, q, 0, q, need - 4, None) == 4
    assert L.qf_lora_adapter_grads(G, A, B, 3072, 3072, 16, None, q, 0, q, need, None) == 1
    assert L.qf_lora_adapter_grads(G, A, B, 0, 3072, 16, q, q, 0, q, need, None) == 0          # empty


def test_workspace_size_bounds_every_layout():
    """qf_workspace_size is at least what each concrete call asks for, over ragged shapes,
    ranks and descriptor counts (the layout changes with the launch size)."""
    L = _lib.lib()
    assert L.qf_workspace_size(9, 10, 10, 1) == 0
    assert L.qf_workspace_size(2, 256, 512, 64) == L.qf_linear_backward_workspace(256, 512, 64)
    rng = __import__("numpy").random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 17))
        rows = int(rng.integers(1, 12000))
        cols = 32 * int(rng.integers(1, 300))
        d = (_lib.LoraDesc * n)()
        for i in range(n):
            d[i].rows = int(rng.integers(0, rows + 1))
            d[i].cols = 32 * int(rng.integers(1, cols // 32 + 1))
            d[i].ldw = d[i].cols
            d[i].r = int(rng.integers(1, 17))
            d[i].group = int(rng.integers(0, 64))
        assert L.qf_lora_workspace(ctypes.byref(d), n) <= L.qf_workspace_size(1, rows, cols, n)
        t = (_lib.TensorDesc * n)()
        for i in range(n):
            t[i].rows, t[i].cols = d[i].rows, 16 * int(rng.integers(1, cols // 16 + 1))
            t[i].ldx, t[i].group = t[i].cols, int(rng.integers(0, 64))
        assert L.qf_nvfp4_tensor_scale_workspace(ctypes.byref(t), n) <= L.qf_workspace_size(0, rows, cols, n)


def _moe_descs(experts):
    d = (_lib.LoraDesc * (2 * experts))()
    for e in range(experts):
        for j, (rows, cols) in enumerate(((3072, 3072), (3072, 1536))):
            k = 2 * e + j
            d[k].rows, d[k].cols, d[k].ldw, d[k].r, d[k].group = rows, cols, cols, 16, k
    return d


def test_lora_layout_of_the_moe_launches():
    """The MoE share's launches.  Pass 1: 8 experts per launch (16 matrices, 55,296 tiles of
    32 x 64) run the full grid of 768 workgroups (3 per CU), 18 tiles per wave at most; 2
    experts keep the full grid (5 tiles per wave); one expert's 6,912 tiles take 432
    workgroups of 4 tiles per wave.  Pass 2 (no M): units of a 512-column slab of 32 rows for 8 experts, 16
    rows for 2 and 8 rows for one (units shrink until a launch has 512 workgroups).
    Gradients: 512-row blocks for 8 experts, 256 for one."""
    L = _lib.lib()
    out = (ctypes.c_int32 * 6)()
    tiles = (3072 // 32) * (3072 // 64) + (3072 // 32) * (1536 // 64)
    slabs_rows = lambda rows: (3072 // rows) * 6 + (3072 // rows) * 3      # units per expert
    assert L.qf_lora_layout(ctypes.byref(_moe_descs(8)), 16, out) == 0
    assert tuple(out) == (18, 768, 512, 8 * (6 * 6 + 6 * 3), 32, 8 * slabs_rows(32) // 4)
    assert -(-8 * tiles // (4 * 768)) == 18
    assert L.qf_lora_layout(ctypes.byref(_moe_descs(2)), 4, out) == 0
    assert tuple(out)[:2] == (5, 768) and tuple(out)[4:] == (16, 2 * slabs_rows(16) // 4)
    assert L.qf_lora_layout(ctypes.byref(_moe_descs(1)), 2, out) == 0
    assert tuple(out) == (4, tiles // 16, 256, 12 * 6 + 12 * 3, 8, slabs_rows(8) // 4)
    assert L.qf_lora_layout(ctypes.byref(_moe_descs(1)), 2, None) == 1


def test_noalloc_tensor_scale_refuses_before_any_hip_call():
    """The no-allocation variant checks its arguments and that its partials fit the fixed
    array (16 groups of the persistent grid) before touching the GPU."""
    L = _lib.lib()
    q = _addr(0x10100000)
    d = (_lib.TensorDesc * 1)()
    d[0].x, d[0].rows, d[0].cols, d[0].ldx, d[0].group = 0x10000000, 4096, 4096, 4096, 63
    assert L.qf_noalloc_scratch_bytes() == 4 * 2048 * 16
    assert L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(d), 1, 64, q, None, None) == 4   # 64 x 2048 partials
    assert L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(d), 1, 63, q, None, None) == 7   # group 63 >= 63
    assert L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(d), 1, 64, None, None, None) == 1
    d[0].x = 0x10000002
    assert L.qf_nvfp4_tensor_scale_grouped_noalloc(ctypes.byref(d), 1, 64, q, None, None) == 3


def _moe_experts(k):
    """Two stacked-experts descriptors (gate/up 3072x3072, down 3072x1536, rank 16) of k
    experts each, tied groups 2e and 2e + 1."""
    x = (_lib.LoraExpertsDesc * 2)()
    for j, (rows, cols) in enumerate(((3072, 3072), (3072, 1536))):
        d = x[j].d
        d.W, d.A, d.B = 0x10000000, 0x10200000, 0x10300000
        d.rows, d.cols, d.ldw, d.r, d.group = rows, cols, cols, 16, j
        x[j].count, x[j].group_stride = k, 2
    return x


def test_lora_experts_layout_and_workspace_match_the_grouped_form():
    """k stacked experts per descriptor lay out exactly like the 2k single-expert
    descriptors of the grouped calls (same tiles, units, workgroups and workspace)."""
    L = _lib.lib()
    out_e, out_g = (ctypes.c_int32 * 6)(), (ctypes.c_int32 * 6)()
    for k in (1, 2, 8):
        x = _moe_experts(k)
        assert L.qf_lora_experts_layout(ctypes.byref(x), 2, out_e) == 0
        assert L.qf_lora_layout(ctypes.byref(_moe_descs(k)), 2 * k, out_g) == 0
        assert tuple(out_e) == tuple(out_g)
        assert L.qf_lora_experts_workspace(ctypes.byref(x), 2) == L.qf_lora_workspace(ctypes.byref(_moe_descs(k)), 2 * k)
    # 32 experts in one call: 64 groups, beyond the grouped calls' 16 descriptors
    x = _moe_experts(32)
    assert L.qf_lora_experts_layout(ctypes.byref(x), 2, out_e) == 0
    tiles = 32 * ((3072 // 32) * (3072 // 64) + (3072 // 32) * (1536 // 64))
    assert tuple(out_e)[:2] == (-(-tiles // (4 * 768)), 768)
    assert tuple(out_e)[4:] == (32, 32 * ((3072 // 32) * 6 + (3072 // 32) * 3) // 4)


def test_lora_experts_validation():
    L = _lib.lib()
    q = _addr(0x10100000)
    x = _moe_experts(8)
    need = L.qf_lora_experts_workspace(ctypes.byref(x), 2)
    assert need > 0
    call = lambda n_groups=16, ws=need: L.qf_lora_experts_merge_tensor_scale_nvfp4(ctypes.byref(x), 2, n_groups, q,
                                                                                  None, q, ws, None)
    assert call(ws=need - 4) == 4                                  # workspace too small
    assert call(n_groups=15) == 7                                  # expert 7 of down: group 15
    x[1].count = 0
    assert L.qf_lora_experts_workspace(ctypes.byref(x), 2) == 0
    assert call() == 7
    x[1].count = 8
    x[1].group_stride = -1
    assert call() == 7
    x[1].group_stride = 2
    x[0].count = x[1].count = 33                                   # group 65 >= QF_MAX_GROUPS
    assert call(n_groups=64) == 7
    x[0].count = x[1].count = 8
    x[0].d.M = 0x10400000                                          # no merge scratch here
    assert call() == 7
    assert L.qf_lora_experts_merge_qdq_pack_nvfp4(ctypes.byref(x), 2, q, None) == 7
    x[0].d.M = 0
    assert L.qf_lora_experts_merge_qdq_pack_nvfp4(ctypes.byref(x), 2, q, None) == 1   # no y and no codes
    assert L.qf_lora_experts_adapter_grads(ctypes.byref(x), 2, 0, q, need, None) == 1  # no G, dA, dB
    assert L.qf_lora_experts_adapter_grads(ctypes.byref(x), 17, 0, q, need, None) == 7
    assert L.qf_lora_experts_layout(ctypes.byref(x), 2, None) == 1
