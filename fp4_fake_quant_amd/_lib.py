"""ctypes loader for libqf.so (the gfx950 HIP library built in-tree).

The library must exist: there is no fallback implementation.  Build it with
``python -m fp4_fake_quant_amd.build`` (``__graft_entry__.build()`` does the same).
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqf.so")

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_void_p = ctypes.c_void_p
c_size_t = ctypes.c_size_t
c_u32 = ctypes.c_uint32


class TensorDesc(ctypes.Structure):
    """Mirror of qf_tensor_desc in include/qf.h."""
    _fields_ = [
        ("x", c_void_p),
        ("rows", c_i64), ("cols", c_i64), ("ldx", c_i64),
        ("y", c_void_p),
        ("ldy", c_i64),
        ("codes", c_void_p),
        ("scales", c_void_p),
        ("group", ctypes.c_int32),
    ]


class LoraDesc(ctypes.Structure):
    """Mirror of qf_lora_desc in include/qf.h."""
    _fields_ = [
        ("W", c_void_p),
        ("rows", c_i64), ("cols", c_i64), ("ldw", c_i64),
        ("A", c_void_p), ("B", c_void_p),
        ("r", ctypes.c_int32), ("group", ctypes.c_int32),
        ("M", c_void_p), ("y", c_void_p), ("codes", c_void_p), ("scales", c_void_p),
        ("G", c_void_p), ("dA", c_void_p), ("dB", c_void_p),
    ]


class LoraExpertsDesc(ctypes.Structure):
    """Mirror of qf_lora_experts in include/qf.h."""
    _fields_ = [("d", LoraDesc), ("count", ctypes.c_int32), ("group_stride", ctypes.c_int32)]


class StTensor(ctypes.Structure):
    """Mirror of qf_st_tensor in include/qf.h."""
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_char_p), ("ndim", ctypes.c_int32),
                ("shape", ctypes.POINTER(c_i64)), ("data", c_void_p)]


class GgufTensor(ctypes.Structure):
    """Mirror of qf_gguf_tensor in include/qf.h."""
    _fields_ = [("name", ctypes.c_char_p), ("ndim", ctypes.c_int32), ("dims", ctypes.POINTER(c_i64)),
                ("type", ctypes.c_uint32), ("data", c_void_p), ("nbytes", ctypes.c_uint64)]


# name -> (restype, argtypes); every entry point declared in include/qf.h
SIGNATURES = {
    "qf_version": (c_u32, []),
    "qf_status_str": (ctypes.c_char_p, [c_int]),
    "qf_last_hip_error": (c_int, []),
    "qf_packed_bytes": (c_size_t, [c_int, c_i64, c_i64]),
    "qf_nvfp4_tensor_scale_workspace": (c_size_t, [c_void_p, c_int]),
    "qf_nvfp4_tensor_scale_grouped": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qf_nvfp4_tensor_scale_tracked": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_size_t, c_void_p]),
    "qf_nvfp4_tensor_scale": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qf_workspace_size": (c_size_t, [c_int, c_i64, c_i64, c_int]),
    "qf_qdq_nvfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p]),
    "qf_pack_nvfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_void_p, c_void_p]),
    "qf_qdq_pack_nvfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p, c_void_p, c_void_p]),
    "qf_qdq_pack_nvfp4_grouped": (c_int, [c_void_p, c_int, c_void_p, c_void_p]),
    "qf_qdq_mxfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_i64, c_void_p]),
    "qf_pack_mxfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_void_p]),
    "qf_qdq_pack_mxfp4": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_i64, c_void_p, c_void_p, c_void_p]),
    "qf_qdq_pack_mxfp4_grouped": (c_int, [c_void_p, c_int, c_void_p]),
    "qf_qdq_q4k": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_i64, c_void_p]),
    "qf_pack_q4k": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p]),
    "qf_qdq_pack_q4k": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_i64, c_void_p, c_void_p]),
    "qf_qdq_pack_q4k_grouped": (c_int, [c_void_p, c_int, c_void_p]),
    "qf_ste_backward": (c_int, [c_void_p, c_void_p, c_i64, c_int, c_void_p]),
    "qf_selftest_conversions": (c_int, [c_void_p, c_void_p]),
    "qf_lora_workspace": (c_size_t, [c_void_p, c_int]),
    "qf_lora_layout": (c_int, [c_void_p, c_int, c_void_p]),
    "qf_lora_merge_tensor_scale_nvfp4_grouped": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                                         c_size_t, c_void_p]),
    "qf_lora_merge_qdq_pack_nvfp4_grouped": (c_int, [c_void_p, c_int, c_void_p, c_void_p]),
    "qf_lora_adapter_grads_grouped": (c_int, [c_void_p, c_int, c_int, c_void_p, c_size_t, c_void_p]),
    "qf_lora_experts_workspace": (c_size_t, [c_void_p, c_int]),
    "qf_lora_experts_layout": (c_int, [c_void_p, c_int, c_void_p]),
    "qf_lora_experts_merge_tensor_scale_nvfp4": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                                         c_size_t, c_void_p]),
    "qf_lora_experts_merge_qdq_pack_nvfp4": (c_int, [c_void_p, c_int, c_void_p, c_void_p]),
    "qf_lora_experts_adapter_grads": (c_int, [c_void_p, c_int, c_int, c_void_p, c_size_t, c_void_p]),
    "qf_lora_merge_tensor_scale_nvfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_int, c_void_p,
                                                 c_void_p, c_size_t, c_void_p]),
    "qf_lora_merge_qdq_pack_nvfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_int, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p]),
    "qf_lora_adapter_grads": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_int, c_void_p, c_void_p, c_int,
                                      c_void_p, c_size_t, c_void_p]),
    "qf_gemm_mxfp4": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64, c_i64, c_i64, c_i64, ctypes.c_uint, c_void_p]),
    "qf_gemm_mxfp4_packed": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p]),
    "qf_gemm_mxfp4_packed_w": (c_int, [c_void_p, c_i64, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p]),
    "qf_qdq_pack_mxfp4_rule": (c_int, [c_void_p, c_int, c_int, c_void_p]),
    "qf_qdq_pack_q4k_rule": (c_int, [c_void_p, c_int, c_int, c_void_p]),
    "qf_dequant_nvfp4": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p]),
    "qf_dequant_mxfp4": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_i64, c_void_p]),
    "qf_dequant_q4k": (c_int, [c_void_p, c_i64, c_i64, c_void_p, c_i64, c_void_p]),
    "qf_transpose_bf16": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_i64, c_int, c_void_p]),
    "qf_linear_backward_workspace": (c_size_t, [c_i64, c_i64, c_i64]),
    "qf_linear_backward_mxfp4": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64,
                                         c_void_p, c_i64, c_i64, c_i64, c_i64, ctypes.c_uint, c_void_p, c_size_t,
                                         c_void_p]),
    "qf_gemm_nvfp4": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64, c_i64, c_i64, c_i64, ctypes.c_uint,
                              c_void_p, c_void_p, c_void_p]),
    "qf_ste_backward_clipped_nvfp4": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_int,
                                              c_void_p]),
    "qf_ste_backward_clipped_mxfp4": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_i64, c_int, c_void_p, c_int,
                                              c_void_p]),
    "qf_linear_forward_mxfp4": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64, c_i64, c_i64, c_i64,
                                        ctypes.c_uint, c_void_p, c_i64, c_void_p, c_i64, c_void_p]),
    "qf_noalloc_scratch_bytes": (c_size_t, []),
    "qf_nvfp4_tensor_scale_grouped_noalloc": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "qf_write_safetensors": (c_int, [ctypes.c_char_p, c_void_p, c_int, c_void_p, c_void_p, c_int]),
    "qf_write_gguf": (c_int, [ctypes.c_char_p, c_void_p, c_int, c_void_p, c_void_p, c_int]),
    "qf_linear_forward_nvfp4": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_void_p, c_i64, c_i64, c_i64, c_i64,
                                        ctypes.c_uint, c_void_p, c_void_p, c_void_p, c_i64, c_void_p, c_i64,
                                        c_void_p]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_fake_quant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib
