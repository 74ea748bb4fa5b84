"""Python binding of libqf (include/qf.h): MI355X simulated quantization.

Argument marshalling only.  Each function has the name of the C entry point
it calls, takes torch tensors that live on the GPU (bf16 data as
torch.bfloat16, packed bytes as torch.uint8, scales as torch.float32),
passes their device pointers, sizes and strides plus torch's current HIP
stream, and raises QFError on a non-zero status.  Outputs that are not
given are allocated with torch (device memory is torch's job here); every
computation runs in the library's HIP kernels.
"""

import ctypes

import torch

from ._lib import GgufTensor, LoraDesc, LoraExpertsDesc, StTensor, TensorDesc, lib

QF_OK = 0
QF_QDQ_A, QF_QDQ_W, QF_FP4_CORES, QF_MX_NOCLIP = 1, 2, 4, 8
QF_FMT_NVFP4, QF_FMT_MXFP4, QF_FMT_Q4K = 0, 1, 2
QF_OP_NVFP4_TENSOR_SCALE, QF_OP_LORA, QF_OP_LINEAR_BACKWARD = 0, 1, 2
MAX_GROUPED = 16
BLOCK = {QF_FMT_NVFP4: 16, QF_FMT_MXFP4: 32, QF_FMT_Q4K: 256}


class QFError(RuntimeError):
    def __init__(self, status, where):
        msg = lib().qf_status_str(status).decode()
        if status == 5:
            msg += f" (hipError {lib().qf_last_hip_error()})"
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status, where):
    if status != QF_OK:
        raise QFError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _mat(x, name):
    """rows, cols, row stride of a 2-D tensor with unit column stride."""
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return x.shape[0], x.shape[1], x.stride(0) if x.shape[0] > 1 else max(x.shape[1], x.stride(0))


def _bf16(x, name):
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16")
    return x


def _out_like(x, y):
    return torch.empty(x.shape, dtype=torch.bfloat16, device=x.device) if y is None else _bf16(y, "y")


def _packed(fmt, rows, cols, device, codes, scales):
    if codes is None:
        codes = torch.empty((rows, cols // 2) if fmt != QF_FMT_Q4K else (rows, cols // 256, 144),
                            dtype=torch.uint8, device=device)
    if scales is None and fmt != QF_FMT_Q4K:
        scales = torch.empty((rows, cols // BLOCK[fmt]), dtype=torch.uint8, device=device)
    return codes, scales


# ------------------------------------------------------------ helpers ----
def qf_version():
    v = lib().qf_version()
    return (v >> 16, (v >> 8) & 0xFF, v & 0xFF)


def qf_packed_bytes(fmt, rows, cols):
    return lib().qf_packed_bytes(fmt, rows, cols)


def _descs(items):
    n = len(items)
    arr = (TensorDesc * max(n, 1))()
    for i, it in enumerate(items):
        x = _bf16(it["x"], "x")
        rows, cols, ldx = _mat(x, "x")
        d = arr[i]
        d.x, d.rows, d.cols, d.ldx = x.data_ptr(), rows, cols, ldx
        y = it.get("y")
        if y is not None:
            _bf16(y, "y")
            d.y, d.ldy = y.data_ptr(), _mat(y, "y")[2]
        d.codes = it["codes"].data_ptr() if it.get("codes") is not None else None
        d.scales = it["scales"].data_ptr() if it.get("scales") is not None else None
        d.group = int(it.get("group", 0))
    return arr, n


# --------------------------------------------------- NVFP4 tensor scale ---
def qf_nvfp4_tensor_scale_workspace(items):
    arr, n = _descs(items)
    return lib().qf_nvfp4_tensor_scale_workspace(ctypes.byref(arr), n)


def qf_nvfp4_tensor_scale_grouped(items, n_groups, d_scales=None, d_nonfinite=None, ws=None):
    """items: list of dict(x=bf16 tensor, group=int).  Returns the device float32 scales."""
    dev = items[0]["x"].device if items else torch.device("cuda")
    arr, n = _descs(items)
    need = lib().qf_nvfp4_tensor_scale_workspace(ctypes.byref(arr), n)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    if d_scales is None:
        d_scales = torch.empty(n_groups, dtype=torch.float32, device=dev)
    _check(lib().qf_nvfp4_tensor_scale_grouped(ctypes.byref(arr), n, n_groups, _p(d_scales), _p(d_nonfinite),
                                                _p(ws), ws.numel() * ws.element_size(), _stream()),
           "qf_nvfp4_tensor_scale_grouped")
    return d_scales


def qf_nvfp4_tensor_scale_tracked(items, n_groups, d_amax, d_scales=None, d_nonfinite=None, ws=None):
    """Tensor scales from the running maximum d_amax (device float32 [n_groups], updated in
    place: max(d_amax, this call's group maxima)); items as qf_nvfp4_tensor_scale_grouped."""
    if d_amax.dtype != torch.float32 or d_amax.device.type != "cuda" or d_amax.numel() < n_groups:
        raise TypeError("d_amax must be a float32 device tensor with a value per group")
    dev = items[0]["x"].device if items else d_amax.device
    arr, n = _descs(items)
    need = lib().qf_nvfp4_tensor_scale_workspace(ctypes.byref(arr), n)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    if d_scales is None:
        d_scales = torch.empty(n_groups, dtype=torch.float32, device=dev)
    _check(lib().qf_nvfp4_tensor_scale_tracked(ctypes.byref(arr), n, n_groups, _p(d_amax), _p(d_scales),
                                                _p(d_nonfinite), _p(ws), ws.numel() * ws.element_size(), _stream()),
           "qf_nvfp4_tensor_scale_tracked")
    return d_scales


def qf_workspace_size(op, rows, cols, n):
    return lib().qf_workspace_size(int(op), int(rows), int(cols), int(n))


def qf_nvfp4_tensor_scale(x, d_scale=None, d_nonfinite=None, ws=None):
    """Tensor scale of one tied group: x is a bf16 tensor or a list of them (e.g. Q, K, V).
    Contiguous members go through the pointer-array call, strided ones through the grouped
    call (same arithmetic).  Returns the device float32 scale (shape [1])."""
    xs = list(x) if isinstance(x, (list, tuple)) else [x]
    if not all(t.is_contiguous() for t in xs):
        return qf_nvfp4_tensor_scale_grouped([dict(x=t, group=0) for t in xs], 1, d_scale, d_nonfinite, ws)
    dev = xs[0].device if xs else torch.device("cuda")
    ptrs = (ctypes.c_void_p * max(len(xs), 1))(*[_bf16(t, "x").data_ptr() for t in xs])
    numel = (ctypes.c_int64 * max(len(xs), 1))(*[t.numel() for t in xs])
    need = lib().qf_workspace_size(QF_OP_NVFP4_TENSOR_SCALE, 1, max([t.numel() for t in xs] + [0]), len(xs))
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    if d_scale is None:
        d_scale = torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib().qf_nvfp4_tensor_scale(ptrs, numel, len(xs), _p(d_scale), _p(d_nonfinite), _p(ws),
                                       ws.numel() * ws.element_size(), _stream()), "qf_nvfp4_tensor_scale")
    return d_scale


# ------------------------------------------------------------ QDQ/pack ----
def qf_qdq_nvfp4(x, d_scale, y=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    _check(lib().qf_qdq_nvfp4(_p(x), rows, cols, ldx, _p(d_scale), _p(y), _mat(y, "y")[2], _stream()), "qf_qdq_nvfp4")
    return y


def qf_pack_nvfp4(x, d_scale, codes=None, scales=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    codes, scales = _packed(QF_FMT_NVFP4, rows, cols, x.device, codes, scales)
    _check(lib().qf_pack_nvfp4(_p(x), rows, cols, ldx, _p(d_scale), _p(codes), _p(scales), _stream()), "qf_pack_nvfp4")
    return codes, scales


def qf_qdq_pack_nvfp4(x, d_scale, y=None, codes=None, scales=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    codes, scales = _packed(QF_FMT_NVFP4, rows, cols, x.device, codes, scales)
    _check(lib().qf_qdq_pack_nvfp4(_p(x), rows, cols, ldx, _p(d_scale), _p(y), _mat(y, "y")[2], _p(codes), _p(scales),
                                   _stream()), "qf_qdq_pack_nvfp4")
    return y, codes, scales


def qf_qdq_pack_nvfp4_grouped(items, d_scales):
    """items: list of dict(x, y=None, codes=None, scales=None, group)."""
    arr, n = _descs(items)
    _check(lib().qf_qdq_pack_nvfp4_grouped(ctypes.byref(arr), n, _p(d_scales), _stream()), "qf_qdq_pack_nvfp4_grouped")


def qf_qdq_mxfp4(x, y=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    _check(lib().qf_qdq_mxfp4(_p(x), rows, cols, ldx, _p(y), _mat(y, "y")[2], _stream()), "qf_qdq_mxfp4")
    return y


def qf_pack_mxfp4(x, codes=None, scales=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    codes, scales = _packed(QF_FMT_MXFP4, rows, cols, x.device, codes, scales)
    _check(lib().qf_pack_mxfp4(_p(x), rows, cols, ldx, _p(codes), _p(scales), _stream()), "qf_pack_mxfp4")
    return codes, scales


def qf_qdq_pack_mxfp4(x, y=None, codes=None, scales=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    codes, scales = _packed(QF_FMT_MXFP4, rows, cols, x.device, codes, scales)
    _check(lib().qf_qdq_pack_mxfp4(_p(x), rows, cols, ldx, _p(y), _mat(y, "y")[2], _p(codes), _p(scales), _stream()),
           "qf_qdq_pack_mxfp4")
    return y, codes, scales


def qf_qdq_pack_mxfp4_grouped(items):
    arr, n = _descs(items)
    _check(lib().qf_qdq_pack_mxfp4_grouped(ctypes.byref(arr), n, _stream()), "qf_qdq_pack_mxfp4_grouped")


def qf_qdq_q4k(x, y=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    _check(lib().qf_qdq_q4k(_p(x), rows, cols, ldx, _p(y), _mat(y, "y")[2], _stream()), "qf_qdq_q4k")
    return y


def qf_pack_q4k(x, blocks=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    blocks, _ = _packed(QF_FMT_Q4K, rows, cols, x.device, blocks, None)
    _check(lib().qf_pack_q4k(_p(x), rows, cols, ldx, _p(blocks), _stream()), "qf_pack_q4k")
    return blocks


def qf_qdq_pack_q4k(x, y=None, blocks=None):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    y = _out_like(x, y)
    blocks, _ = _packed(QF_FMT_Q4K, rows, cols, x.device, blocks, None)
    _check(lib().qf_qdq_pack_q4k(_p(x), rows, cols, ldx, _p(y), _mat(y, "y")[2], _p(blocks), _stream()), "qf_qdq_pack_q4k")
    return y, blocks


QF_MX_RULE_FLOOR, QF_MX_RULE_NOCLIP = 0, 1


def qf_qdq_pack_mxfp4_rule(items, rule):
    """qf_qdq_pack_mxfp4_grouped under shared-exponent rule QF_MX_RULE_FLOOR or QF_MX_RULE_NOCLIP."""
    arr, n = _descs(items)
    _check(lib().qf_qdq_pack_mxfp4_rule(ctypes.byref(arr), n, int(rule), _stream()), "qf_qdq_pack_mxfp4_rule")


QF_Q4K_RULE_MINMAX, QF_Q4K_RULE_MSE = 0, 1


def qf_qdq_pack_q4k_rule(items, rule):
    """qf_qdq_pack_q4k_grouped under sub-block scale rule QF_Q4K_RULE_MINMAX or QF_Q4K_RULE_MSE."""
    arr, n = _descs(items)
    _check(lib().qf_qdq_pack_q4k_rule(ctypes.byref(arr), n, int(rule), _stream()), "qf_qdq_pack_q4k_rule")


def qf_qdq_pack_q4k_grouped(items):
    arr, n = _descs(items)
    _check(lib().qf_qdq_pack_q4k_grouped(ctypes.byref(arr), n, _stream()), "qf_qdq_pack_q4k_grouped")


# ----------------------------------------------------------------- STE ----
def qf_ste_backward(g_q, g_latent=None, accumulate=False):
    _bf16(g_q, "g_q")
    if not g_q.is_contiguous():
        raise ValueError("g_q must be contiguous")
    if g_latent is None:
        g_latent = torch.empty(g_q.shape, dtype=torch.float32, device=g_q.device)
    if g_latent.dtype != torch.float32 or not g_latent.is_contiguous() or g_latent.numel() != g_q.numel():
        raise ValueError("g_latent must be a contiguous float32 tensor with g_q's element count")
    _check(lib().qf_ste_backward(_p(g_q), _p(g_latent), g_q.numel(), int(bool(accumulate)), _stream()), "qf_ste_backward")
    return g_latent


def _ste_clip_args(g_q, x, g_latent):
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    _bf16(g_q, "g_q")
    if tuple(g_q.shape) != (rows, cols) or not g_q.is_contiguous():
        raise ValueError("g_q must be a contiguous tensor of x's shape")
    if g_latent is None:
        g_latent = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    if g_latent.dtype != torch.float32 or tuple(g_latent.shape) != (rows, cols) or not g_latent.is_contiguous():
        raise ValueError("g_latent must be a contiguous float32 tensor of x's shape")
    return rows, cols, ldx, g_latent


def qf_ste_backward_clipped_nvfp4(g_q, x, d_scale, g_latent=None, accumulate=False):
    """g_latent = f32(g_q), or +0.0 where the NVFP4 quantizer (tensor scale d_scale)
    saturated x; added to g_latent when accumulate."""
    rows, cols, ldx, g_latent = _ste_clip_args(g_q, x, g_latent)
    _check(lib().qf_ste_backward_clipped_nvfp4(_p(g_q), _p(x), rows, cols, ldx, _p(d_scale), _p(g_latent),
                                               int(bool(accumulate)), _stream()), "qf_ste_backward_clipped_nvfp4")
    return g_latent


def qf_ste_backward_clipped_mxfp4(g_q, x, g_latent=None, accumulate=False, rule=QF_MX_RULE_FLOOR):
    """g_latent = f32(g_q), or +0.0 where the MXFP4 quantizer (shared-exponent rule `rule`)
    saturated x; added to g_latent when accumulate."""
    rows, cols, ldx, g_latent = _ste_clip_args(g_q, x, g_latent)
    _check(lib().qf_ste_backward_clipped_mxfp4(_p(g_q), _p(x), rows, cols, ldx, int(rule), _p(g_latent),
                                               int(bool(accumulate)), _stream()), "qf_ste_backward_clipped_mxfp4")
    return g_latent


# ---------------------------------------------------------------- LoRA ----
class LoraBatch:
    """Descriptor array for the qf_lora_* calls, built once and reusable.

    items: list of dict(W, A, B, group, M=None, y=None, codes=None, scales=None,
    G=None, dA=None, dB=None) of device tensors; W [rows, cols] bf16 with contiguous
    rows, A [r, cols] and B [rows, r] contiguous bf16.  The tensors must stay alive
    (and keep their storage) while the batch is used.
    """

    def __init__(self, items):
        self.items = items
        self.arr = (LoraDesc * max(len(items), 1))()
        self.n = len(items)
        self.device = items[0]["W"].device if items else torch.device("cuda")
        for i, it in enumerate(items):
            W = _bf16(it["W"], "W")
            rows, cols, ldw = _mat(W, "W")
            A, B = _bf16(it["A"], "A"), _bf16(it["B"], "B")
            if A.dim() != 2 or B.dim() != 2 or not A.is_contiguous() or not B.is_contiguous():
                raise ValueError("A [r, cols] and B [rows, r] must be contiguous 2-D tensors")
            r = A.shape[0]
            if A.shape[1] != cols or tuple(B.shape) != (rows, r):
                raise ValueError(f"adapter shapes {tuple(A.shape)}, {tuple(B.shape)} do not fit W {rows}x{cols}")
            d = self.arr[i]
            d.W, d.rows, d.cols, d.ldw = W.data_ptr(), rows, cols, ldw
            d.A, d.B, d.r, d.group = A.data_ptr(), B.data_ptr(), r, int(it.get("group", 0))
            for name in ("M", "y", "codes", "scales", "G", "dA", "dB"):
                t = it.get(name)
                if t is not None and not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous")
                setattr(d, name, t.data_ptr() if t is not None else None)
        self.ref = ctypes.byref(self.arr)
        self.workspace_bytes = lib().qf_lora_workspace(self.ref, self.n)


def _batch(items):
    return items if isinstance(items, LoraBatch) else LoraBatch(items)


def _lora_ws(b, ws):
    if ws is None:
        ws = torch.empty(max(b.workspace_bytes, 4), dtype=torch.uint8, device=b.device)
    return ws


def qf_lora_workspace(items):
    return _batch(items).workspace_bytes


def qf_lora_layout(items):
    """(most pass-1 tiles per wave, pass-1 workgroups, rows per gradient workgroup, gradient
    workgroups, rows per pass-2 unit, pass-2 workgroups) the LoRA calls choose for these
    descriptors (a host query)."""
    b = _batch(items)
    out = (ctypes.c_int32 * 6)()
    _check(lib().qf_lora_layout(b.ref, b.n, out), "qf_lora_layout")
    return tuple(out)


def qf_lora_merge_tensor_scale_nvfp4_grouped(items, n_groups, d_scales=None, d_nonfinite=None, ws=None):
    b = _batch(items)
    ws = _lora_ws(b, ws)
    if d_scales is None:
        d_scales = torch.empty(n_groups, dtype=torch.float32, device=b.device)
    _check(lib().qf_lora_merge_tensor_scale_nvfp4_grouped(b.ref, b.n, n_groups, _p(d_scales), _p(d_nonfinite),
                                                           _p(ws), ws.numel() * ws.element_size(), _stream()),
           "qf_lora_merge_tensor_scale_nvfp4_grouped")
    return d_scales


def qf_lora_merge_qdq_pack_nvfp4_grouped(items, d_scales):
    b = _batch(items)
    _check(lib().qf_lora_merge_qdq_pack_nvfp4_grouped(b.ref, b.n, _p(d_scales), _stream()),
           "qf_lora_merge_qdq_pack_nvfp4_grouped")


def qf_lora_adapter_grads_grouped(items, accumulate=False, ws=None):
    b = _batch(items)
    ws = _lora_ws(b, ws)
    _check(lib().qf_lora_adapter_grads_grouped(b.ref, b.n, int(bool(accumulate)), _p(ws),
                                               ws.numel() * ws.element_size(), _stream()),
           "qf_lora_adapter_grads_grouped")


class LoraExperts:
    """Stacked-experts descriptors for the qf_lora_experts_* calls, built once and reusable.

    items: list of dict(W, A, B, group, group_stride=1, y=None, codes=None, scales=None,
    G=None, dA=None, dB=None) of contiguous device tensors with a leading expert axis:
    W [E, rows, cols] bf16, A [E, r, cols], B [E, rows, r], y [E, rows, cols],
    codes [E, rows, cols/2], scales [E, rows, cols/16], G [E, rows, cols],
    dA [E, r, cols] and dB [E, rows, r] float32.  Expert e's tied group is
    group + e * group_stride.  There is no merge scratch (M).
    """

    def __init__(self, items):
        self.items = items
        self.arr = (LoraExpertsDesc * max(len(items), 1))()
        self.n = len(items)
        self.device = items[0]["W"].device if items else torch.device("cuda")
        for i, it in enumerate(items):
            W, A, B = _bf16(it["W"], "W"), _bf16(it["A"], "A"), _bf16(it["B"], "B")
            for t, name in ((W, "W"), (A, "A"), (B, "B")):
                if t.dim() != 3 or not t.is_contiguous():
                    raise ValueError(f"{name} must be a contiguous 3-D tensor [experts, ...]")
            E, rows, cols = W.shape
            r = A.shape[1]
            if tuple(A.shape) != (E, r, cols) or tuple(B.shape) != (E, rows, r):
                raise ValueError(f"adapter shapes {tuple(A.shape)}, {tuple(B.shape)} do not fit W {tuple(W.shape)}")
            x = self.arr[i]
            d = x.d
            d.W, d.rows, d.cols, d.ldw = W.data_ptr(), rows, cols, cols
            d.A, d.B, d.r, d.group = A.data_ptr(), B.data_ptr(), r, int(it.get("group", 0))
            d.M = None
            for name in ("y", "codes", "scales", "G", "dA", "dB"):
                t = it.get(name)
                if t is not None and (not t.is_contiguous() or t.shape[0] != E):
                    raise ValueError(f"{name} must be contiguous with {E} experts")
                setattr(d, name, t.data_ptr() if t is not None else None)
            x.count = E
            x.group_stride = int(it.get("group_stride", 1))
        self.ref = ctypes.byref(self.arr)
        self.workspace_bytes = lib().qf_lora_experts_workspace(self.ref, self.n)


def qf_lora_experts_layout(ex):
    """The launch layout of the stacked-experts calls (as qf_lora_layout)."""
    out = (ctypes.c_int32 * 6)()
    _check(lib().qf_lora_experts_layout(ex.ref, ex.n, out), "qf_lora_experts_layout")
    return tuple(out)


def qf_lora_experts_merge_tensor_scale_nvfp4(ex, n_groups, d_scales=None, d_nonfinite=None, ws=None):
    ws = _lora_ws(ex, ws)
    if d_scales is None:
        d_scales = torch.empty(n_groups, dtype=torch.float32, device=ex.device)
    _check(lib().qf_lora_experts_merge_tensor_scale_nvfp4(ex.ref, ex.n, n_groups, _p(d_scales), _p(d_nonfinite),
                                                           _p(ws), ws.numel() * ws.element_size(), _stream()),
           "qf_lora_experts_merge_tensor_scale_nvfp4")
    return d_scales


def qf_lora_experts_merge_qdq_pack_nvfp4(ex, d_scales):
    _check(lib().qf_lora_experts_merge_qdq_pack_nvfp4(ex.ref, ex.n, _p(d_scales), _stream()),
           "qf_lora_experts_merge_qdq_pack_nvfp4")


def qf_lora_experts_adapter_grads(ex, accumulate=False, ws=None):
    ws = _lora_ws(ex, ws)
    _check(lib().qf_lora_experts_adapter_grads(ex.ref, ex.n, int(bool(accumulate)), _p(ws),
                                               ws.numel() * ws.element_size(), _stream()),
           "qf_lora_experts_adapter_grads")


def _lora_single(W, A, B):
    for t, name in ((W, "W"), (A, "A"), (B, "B")):
        if not _bf16(t, name).is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D bf16 tensor")
    rows, cols = W.shape
    r = A.shape[0]
    if A.shape[1] != cols or tuple(B.shape) != (rows, r):
        raise ValueError(f"adapter shapes {tuple(A.shape)}, {tuple(B.shape)} do not fit W {rows}x{cols}")
    return rows, cols, r


def _lora_single_ws(rows, cols, device, ws):
    if ws is None:
        ws = torch.empty(max(lib().qf_workspace_size(QF_OP_LORA, rows, cols, 1), 4), dtype=torch.uint8,
                         device=device)
    return ws


def qf_lora_merge_tensor_scale_nvfp4(W, A, B, d_scale=None, ws=None):
    """NVFP4 tensor scale of M = W + B.A for one contiguous matrix, merged in registers."""
    rows, cols, r = _lora_single(W, A, B)
    ws = _lora_single_ws(rows, cols, W.device, ws)
    if d_scale is None:
        d_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    _check(lib().qf_lora_merge_tensor_scale_nvfp4(_p(W), _p(A), _p(B), rows, cols, r, _p(d_scale), _p(ws),
                                                   ws.numel() * ws.element_size(), _stream()),
           "qf_lora_merge_tensor_scale_nvfp4")
    return d_scale


def qf_lora_merge_qdq_pack_nvfp4(W, A, B, d_scale, y=None, codes=None, scales=None):
    """(y, codes, scales): NVFP4 QDQ + pack of M = W + B.A (merged again in registers)."""
    rows, cols, r = _lora_single(W, A, B)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=W.device) if y is None else y
    codes, scales = _packed(QF_FMT_NVFP4, rows, cols, W.device, codes, scales)
    _check(lib().qf_lora_merge_qdq_pack_nvfp4(_p(W), _p(A), _p(B), rows, cols, r, _p(d_scale), _p(y), _p(codes),
                                               _p(scales), _stream()), "qf_lora_merge_qdq_pack_nvfp4")
    return y, codes, scales


def qf_lora_adapter_grads(G, A, B, dA=None, dB=None, accumulate=False, ws=None):
    """(dA [r, cols], dB [rows, r]) fp32 = (B^T . G, G . A^T) for one contiguous matrix."""
    rows, cols, r = _lora_single(G, A, B)
    ws = _lora_single_ws(rows, cols, G.device, ws)
    dA = torch.empty((r, cols), dtype=torch.float32, device=G.device) if dA is None else dA
    dB = torch.empty((rows, r), dtype=torch.float32, device=G.device) if dB is None else dB
    _check(lib().qf_lora_adapter_grads(_p(G), _p(A), _p(B), rows, cols, r, _p(dA), _p(dB), int(bool(accumulate)),
                                       _p(ws), ws.numel() * ws.element_size(), _stream()), "qf_lora_adapter_grads")
    return dA, dB


# ------------------------------------------------------------- dequant ----
def _dequant_out(rows, cols, device, y):
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    _bf16(y, "y")
    if tuple(y.shape) != (rows, cols):
        raise ValueError(f"y has shape {tuple(y.shape)}, want {(rows, cols)}")
    return y


def _u8(t, name):
    if t.dtype != torch.uint8 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous uint8 tensor")
    return t


def qf_dequant_nvfp4(codes, scales, d_scale, y=None):
    """bf16 [rows, cols] from NVFP4 codes [rows, cols/2] and E4M3 scales [rows, cols/16]."""
    rows, cols = _u8(codes, "codes").shape[0], codes.shape[1] * 2
    y = _dequant_out(rows, cols, codes.device, y)
    _check(lib().qf_dequant_nvfp4(_p(codes), _p(_u8(scales, "scales")), rows, cols, _p(d_scale), _p(y),
                                  _mat(y, "y")[2], _stream()), "qf_dequant_nvfp4")
    return y


def qf_dequant_mxfp4(codes, scales, y=None):
    """bf16 [rows, cols] from MXFP4 codes [rows, cols/2] and E8M0 scales [rows, cols/32]."""
    rows, cols = _u8(codes, "codes").shape[0], codes.shape[1] * 2
    y = _dequant_out(rows, cols, codes.device, y)
    _check(lib().qf_dequant_mxfp4(_p(codes), _p(_u8(scales, "scales")), rows, cols, _p(y), _mat(y, "y")[2],
                                  _stream()), "qf_dequant_mxfp4")
    return y


def qf_dequant_q4k(blocks, rows, cols, y=None):
    """bf16 [rows, cols] from Q4_K blocks (rows * cols / 256 blocks of 144 bytes)."""
    _u8(blocks, "blocks")
    if blocks.numel() != rows * (cols // 256) * 144:
        raise ValueError("blocks do not match rows x cols")
    y = _dequant_out(rows, cols, blocks.device, y)
    _check(lib().qf_dequant_q4k(_p(blocks), rows, cols, _p(y), _mat(y, "y")[2], _stream()), "qf_dequant_q4k")
    return y


# ---------------------------------------------------------------- GEMM ----
def qf_gemm_mxfp4(X, W, Y=None, flags=QF_QDQ_A | QF_QDQ_W):
    """Y[M, N] = QDQ(X)[M, K] . QDQ(W)[N, K]^T (bf16 in, fp32 accumulate, bf16 out)."""
    M, K, ldx = _mat(_bf16(X, "X"), "X")
    N, K2, ldw = _mat(_bf16(W, "W"), "W")
    if K2 != K:
        raise ValueError(f"X has K={K} but W has K={K2}")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _bf16(Y, "Y")
    _check(lib().qf_gemm_mxfp4(_p(X), ldx, _p(W), ldw, _p(Y), _mat(Y, "Y")[2], M, N, K, int(flags), _stream()),
           "qf_gemm_mxfp4")
    return Y


def qf_gemm_nvfp4(X, W, d_scale_x, d_scale_w, Y=None, flags=QF_QDQ_A | QF_QDQ_W):
    """Y[M, N] = QDQ(X) . QDQ(W)^T on the NVFP4 grid with the device fp32 tensor scales
    d_scale_x, d_scale_w (one element each; None for an operand that is not quantized)."""
    M, K, ldx = _mat(_bf16(X, "X"), "X")
    N, K2, ldw = _mat(_bf16(W, "W"), "W")
    if K2 != K:
        raise ValueError(f"X has K={K} but W has K={K2}")
    for t, name in ((d_scale_x, "d_scale_x"), (d_scale_w, "d_scale_w")):
        if t is not None and (t.dtype != torch.float32 or t.device.type != "cuda"):
            raise TypeError(f"{name} must be a float32 device tensor")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _bf16(Y, "Y")
    _check(lib().qf_gemm_nvfp4(_p(X), ldx, _p(W), ldw, _p(Y), _mat(Y, "Y")[2], M, N, K, int(flags), _p(d_scale_x),
                               _p(d_scale_w), _stream()), "qf_gemm_nvfp4")
    return Y


def _linear_forward_args(X, W, Y, Xq, Wq, flags):
    M, K, ldx = _mat(_bf16(X, "X"), "X")
    N, K2, ldw = _mat(_bf16(W, "W"), "W")
    if K2 != K:
        raise ValueError(f"X has K={K} but W has K={K2}")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if Xq is None and flags & QF_QDQ_A:
        Xq = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    if Wq is None and flags & QF_QDQ_W:
        Wq = torch.empty((N, K), dtype=torch.bfloat16, device=X.device)
    _bf16(Y, "Y")
    ldxq = _mat(_bf16(Xq, "Xq"), "Xq")[2] if Xq is not None else 0
    ldwq = _mat(_bf16(Wq, "Wq"), "Wq")[2] if Wq is not None else 0
    return M, N, K, ldx, ldw, Y, Xq, ldxq, Wq, ldwq


def qf_linear_forward_mxfp4(X, W, Y=None, flags=QF_QDQ_A | QF_QDQ_W, Xq=None, Wq=None):
    """(Y, Xq, Wq): Xq = QDQ(X), Wq = QDQ(W) (MXFP4, for the flagged operands), then
    Y = Xq . Wq^T on the BF16 matrix cores; Y equals qf_gemm_mxfp4(X, W, flags) bit for bit."""
    M, N, K, ldx, ldw, Y, Xq, ldxq, Wq, ldwq = _linear_forward_args(X, W, Y, Xq, Wq, flags)
    _check(lib().qf_linear_forward_mxfp4(_p(X), ldx, _p(W), ldw, _p(Y), _mat(Y, "Y")[2], M, N, K, int(flags),
                                         _p(Xq), ldxq, _p(Wq), ldwq, _stream()), "qf_linear_forward_mxfp4")
    return Y, Xq, Wq


def qf_linear_forward_nvfp4(X, W, d_scale_x, d_scale_w, Y=None, flags=QF_QDQ_A | QF_QDQ_W, Xq=None, Wq=None):
    """(Y, Xq, Wq) as qf_linear_forward_mxfp4 on the NVFP4 grid with the device fp32 tensor
    scales d_scale_x, d_scale_w; Y equals qf_gemm_nvfp4 with the same arguments bit for bit."""
    for t, name in ((d_scale_x, "d_scale_x"), (d_scale_w, "d_scale_w")):
        if t is not None and (t.dtype != torch.float32 or t.device.type != "cuda"):
            raise TypeError(f"{name} must be a float32 device tensor")
    M, N, K, ldx, ldw, Y, Xq, ldxq, Wq, ldwq = _linear_forward_args(X, W, Y, Xq, Wq, flags)
    _check(lib().qf_linear_forward_nvfp4(_p(X), ldx, _p(W), ldw, _p(Y), _mat(Y, "Y")[2], M, N, K, int(flags),
                                         _p(d_scale_x), _p(d_scale_w), _p(Xq), ldxq, _p(Wq), ldwq, _stream()),
           "qf_linear_forward_nvfp4")
    return Y, Xq, Wq


def qf_transpose_bf16(x, y=None, qdq_mxfp4=False, rule=QF_MX_RULE_FLOOR):
    """y [cols, rows] = x^T, MXFP4-QDQ'd along x's rows first (under `rule`) when qdq_mxfp4."""
    rows, cols, ldx = _mat(_bf16(x, "x"), "x")
    if y is None:
        y = torch.empty((cols, rows), dtype=torch.bfloat16, device=x.device)
    _bf16(y, "y")
    _check(lib().qf_transpose_bf16(_p(x), rows, cols, ldx, _p(y), _mat(y, "y")[2], (1 + int(rule == QF_MX_RULE_NOCLIP)) if qdq_mxfp4 else 0, _stream()),
           "qf_transpose_bf16")
    return y


def qf_linear_backward_workspace(M, N, K):
    return lib().qf_linear_backward_workspace(M, N, K)


def qf_linear_backward_mxfp4(X, W, dY, dX=None, dW=None, flags=QF_QDQ_A | QF_QDQ_W, ws=None, want=(True, True)):
    """(dX, dW) of Y = Xq . Wq^T: dX = dY . Wq [M, K], dW = dY^T . Xq [N, K] (bf16)."""
    M, K, ldx = _mat(_bf16(X, "X"), "X")
    N, K2, ldw = _mat(_bf16(W, "W"), "W")
    M2, N2, lddy = _mat(_bf16(dY, "dY"), "dY")
    if K2 != K or M2 != M or N2 != N:
        raise ValueError(f"shapes X {tuple(X.shape)}, W {tuple(W.shape)}, dY {tuple(dY.shape)} do not fit")
    if dX is None and want[0]:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    if dW is None and want[1]:
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=X.device)
    need = lib().qf_linear_backward_workspace(M, N, K)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check(lib().qf_linear_backward_mxfp4(_p(X), ldx, _p(W), ldw, _p(dY), lddy, _p(dX),
                                          _mat(dX, "dX")[2] if dX is not None else 0, _p(dW),
                                          _mat(dW, "dW")[2] if dW is not None else 0, M, N, K, int(flags), _p(ws),
                                          ws.numel(), _stream()), "qf_linear_backward_mxfp4")
    return dX, dW


def qf_gemm_mxfp4_packed_w(X, Wc, Ws, Y=None):
    """Y[M, N] = QDQ(X) . dequant(Wc, Ws)^T on the MXFP4 matrix cores; Wc [N, K/2] and
    Ws [N, K/32] uint8 as qf_pack_mxfp4 writes them (contiguous)."""
    M, K, ldx = _mat(_bf16(X, "X"), "X")
    if Wc.dtype != torch.uint8 or Ws.dtype != torch.uint8 or not Wc.is_contiguous() or not Ws.is_contiguous():
        raise ValueError("Wc and Ws must be contiguous uint8 tensors")
    N = Wc.shape[0]
    if tuple(Wc.shape) != (N, K // 2) or tuple(Ws.shape) != (N, K // 32):
        raise ValueError(f"packed W shapes {tuple(Wc.shape)}, {tuple(Ws.shape)} do not fit K={K}")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _bf16(Y, "Y")
    _check(lib().qf_gemm_mxfp4_packed_w(_p(X), ldx, _p(Wc), _p(Ws), _p(Y), _mat(Y, "Y")[2], M, N, K, _stream()),
           "qf_gemm_mxfp4_packed_w")
    return Y


def qf_gemm_mxfp4_packed(Xc, Xs, Wc, Ws, Y=None):
    """Y[M, N] = dequant(Xc, Xs) . dequant(Wc, Ws)^T on the MXFP4 matrix cores; all four
    arrays uint8 as qf_pack_mxfp4 writes them (contiguous), K a multiple of 128."""
    for name, t in (("Xc", Xc), ("Xs", Xs), ("Wc", Wc), ("Ws", Ws)):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-D uint8 tensor")
    M, N, K = Xc.shape[0], Wc.shape[0], Xc.shape[1] * 2
    if Wc.shape[1] * 2 != K or tuple(Xs.shape) != (M, K // 32) or tuple(Ws.shape) != (N, K // 32):
        raise ValueError("packed operand shapes do not agree")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=Xc.device)
    _bf16(Y, "Y")
    _check(lib().qf_gemm_mxfp4_packed(_p(Xc), _p(Xs), _p(Wc), _p(Ws), _p(Y), _mat(Y, "Y")[2], M, N, K, _stream()),
           "qf_gemm_mxfp4_packed")
    return Y


def qf_selftest_conversions(device="cuda"):
    counts = torch.zeros(8, dtype=torch.int64, device=device)
    _check(lib().qf_selftest_conversions(_p(counts), _stream()), "qf_selftest_conversions")
    return counts


# ------------------------------------------------- checkpoint containers ----
_ST_DTYPE = {torch.uint8: "U8", torch.int8: "I8", torch.bool: "BOOL", torch.float8_e4m3fn: "F8_E4M3",
             torch.float8_e5m2: "F8_E5M2", torch.float8_e8m0fnu: "F8_E8M0", torch.int16: "I16",
             torch.float16: "F16", torch.bfloat16: "BF16", torch.int32: "I32", torch.float32: "F32",
             torch.int64: "I64", torch.float64: "F64"}
_ST_SIZE = {"U8": 1, "I8": 1, "BOOL": 1, "F8_E4M3": 1, "F8_E5M2": 1, "F8_E8M0": 1, "U16": 2, "I16": 2, "F16": 2,
            "BF16": 2, "U32": 4, "I32": 4, "F32": 4, "U64": 8, "I64": 8, "F64": 8}


def _host_bytes(t):
    return t.detach().contiguous().cpu()


def _cstrings(strs):
    arr = (ctypes.c_char_p * max(len(strs), 1))(*[x.encode() for x in strs])
    return arr


def qf_write_safetensors(path, tensors, metadata=None):
    """Write a safetensors file.  tensors: list of (name, tensor, dtype) with tensor on any
    device and dtype a safetensors dtype string or None (taken from the tensor); a uint8
    tensor of E4M3 / E8M0 scale bytes is written as "F8_E4M3" / "F8_E8M0" by naming that
    dtype.  metadata: dict of str -> str."""
    keep = []
    arr = (StTensor * max(len(tensors), 1))()
    for i, (name, t, dt) in enumerate(tensors):
        h = _host_bytes(t)
        dt = dt or _ST_DTYPE.get(h.dtype)
        if dt is None or _ST_SIZE.get(dt) != h.element_size():
            raise TypeError(f"{name}: cannot write a {h.dtype} tensor as {dt}")
        shape = (ctypes.c_int64 * max(h.dim(), 1))(*h.shape)
        keep += [h, shape, name.encode(), dt.encode()]
        arr[i].name, arr[i].dtype, arr[i].ndim = keep[-2], keep[-1], h.dim()
        arr[i].shape = ctypes.cast(shape, ctypes.POINTER(ctypes.c_int64))
        arr[i].data = h.data_ptr() if h.numel() else None
    meta = metadata or {}
    keys, vals = _cstrings(list(meta)), _cstrings([str(v) for v in meta.values()])
    _check(lib().qf_write_safetensors(str(path).encode(), ctypes.byref(arr), len(tensors), keys, vals, len(meta)),
           "qf_write_safetensors")


def qf_write_gguf(path, tensors, kv=None):
    """Write a GGUF-style file.  tensors: list of (name, tensor of raw bytes, dims innermost
    first, type code); kv: dict of str -> str."""
    keep = []
    arr = (GgufTensor * max(len(tensors), 1))()
    for i, (name, t, dims, typ) in enumerate(tensors):
        h = _host_bytes(t)
        d = (ctypes.c_int64 * len(dims))(*dims)
        keep += [h, d, name.encode()]
        arr[i].name, arr[i].ndim = keep[-1], len(dims)
        arr[i].dims = ctypes.cast(d, ctypes.POINTER(ctypes.c_int64))
        arr[i].type, arr[i].data = int(typ), (h.data_ptr() if h.numel() else None)
        arr[i].nbytes = h.numel() * h.element_size()
    kv = kv or {}
    keys, vals = _cstrings(list(kv)), _cstrings([str(v) for v in kv.values()])
    _check(lib().qf_write_gguf(str(path).encode(), ctypes.byref(arr), len(tensors), keys, vals, len(kv)),
           "qf_write_gguf")


GGUF_TYPE_Q4_K = 12
Q4K_BLOCK_LAYOUT = ("144-byte blocks per 256 weights along a row: d (fp16 LE), dmin (fp16 LE), a 96-bit "
                    "little-endian stream with the 6-bit sub-block scale j at bits 6j and min j at bits 48+6j, "
                    "128 code bytes with element 2i in the low nibble and 2i+1 in the high nibble; "
                    "w = d*sc_j*q - dmin*m_j")


def export_fp4_tensors(prefix, fmt, codes, scales, d_scale=None, d_input_scale=None):
    """The (name, tensor, dtype) list of one packed NVFP4 / MXFP4 layer in the names this
    library uses ("compressed-tensors-style"): weight_packed, weight_scale (E4M3 or E8M0
    bytes), and for NVFP4 weight_global_scale (the layer group's dequant multiplier s_t)
    and, when given, input_global_scale (the tracked activation s_t)."""
    out = [(f"{prefix}.weight_packed", codes, "U8"),
           (f"{prefix}.weight_scale", scales, "F8_E4M3" if fmt == QF_FMT_NVFP4 else "F8_E8M0")]
    if fmt == QF_FMT_NVFP4:
        if d_scale is None:
            raise ValueError("NVFP4 needs the tensor scale")
        out.append((f"{prefix}.weight_global_scale", d_scale.reshape(-1)[:1], "F32"))
        if d_input_scale is not None:
            out.append((f"{prefix}.input_global_scale", d_input_scale.reshape(-1)[:1], "F32"))
    return out


def export_q4k_tensor(name, blocks, rows, cols):
    """The (name, bytes, dims, type) entry of one Q4_K matrix for qf_write_gguf."""
    return (name, blocks, (cols, rows), GGUF_TYPE_Q4_K)
