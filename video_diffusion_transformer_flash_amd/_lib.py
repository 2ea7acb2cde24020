"""ctypes declarations of libvdtflash.so (the C ABI in include/vdtflash.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvdtflash.so")

DIT_OK, DIT_EINVAL, DIT_EUNSUPPORTED, DIT_EWORKSPACE, DIT_EHIP = 0, -1, -2, -3, -4
DIT_F32, DIT_BF16, DIT_FP8_E4M3 = 0, 1, 2

c_i32, c_i64, c_f32, c_size, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)


class Dims(ctypes.Structure):
    _fields_ = [("T", c_i32), ("H", c_i32), ("W", c_i32), ("n_text", c_i32), ("n_audio", c_i32),
                ("d_model", c_i32), ("n_heads", c_i32), ("head_dim", c_i32), ("d_ffn", c_i32),
                ("rope_t", c_i32), ("rope_h", c_i32), ("rope_w", c_i32), ("rope_base", c_f32), ("eps", c_f32),
                ("stride", c_i32), ("act_dtype", c_i32), ("w_dtype", c_i32), ("n_ctrl", c_i32),
                ("ctrl_offset", c_i32), ("n_fixed", c_i32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [("g1", c_vp), ("wqkv", c_vp), ("wo", c_vp), ("g2", c_vp), ("wgate", c_vp), ("wup", c_vp),
                ("wdown", c_vp), ("s_wqkv", c_vp), ("s_wo", c_vp), ("s_wgate", c_vp), ("s_wup", c_vp),
                ("s_wdown", c_vp)]


# name -> (restype, argtypes); every symbol declared in include/vdtflash.h
SIGNATURES = {
    "dit_keep_dims": (c_i32, [c_i32, c_i32, c_i32, P_i32, P_i32]),
    "dit_keep_index": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "dit_nearest_kept_map": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "dit_block_workspace_size": (c_i32, [ctypes.POINTER(Dims), c_i32, ctypes.POINTER(c_size)]),
    "dit_block_forward": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, ctypes.POINTER(BlockWeights), c_i32,
                                  c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dit_block_forward_ctrl": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp, c_i32, c_vp,
                                       ctypes.POINTER(BlockWeights), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                       c_size, c_vp]),
    "dit_block_forward_noalloc": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, ctypes.POINTER(BlockWeights), c_i32,
                                          c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "dit_history_count": (c_i32, [c_i32, c_i32, c_i32, P_i32]),
    "dit_history_index": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp]),
    "dit_stack_workspace_size": (c_i32, [ctypes.POINTER(Dims), c_vp, c_i32, ctypes.POINTER(c_size)]),
    "dit_stack_sample": (c_i32, [ctypes.POINTER(Dims), ctypes.POINTER(BlockWeights), c_i32, c_vp, c_i32, c_vp, c_vp,
                                 c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dit_stack_sample_ctrl": (c_i32, [ctypes.POINTER(Dims), ctypes.POINTER(BlockWeights), c_i32, c_vp, c_i32, c_vp,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dit_long_video_workspace_size": (c_i32, [ctypes.POINTER(Dims), c_vp, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "dit_long_video_sample": (c_i32, [ctypes.POINTER(Dims), ctypes.POINTER(BlockWeights), c_i32, c_vp, c_i32, c_vp,
                                      c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dit_quantize_fp8": (c_i32, [c_vp, c_i32, c_i64, c_vp, c_vp, c_vp]),
    "dit_gather_kept": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "dit_broadcast_residual": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "dit_attention_workspace_size": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "dit_attention": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dit_rmsnorm": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_vp, c_vp]),
    "dit_project_residual_workspace_size": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "dit_project_residual": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                                     c_vp]),
    "dit_trace_enable": (c_i32, [c_i32]),
    "dit_trace_count": (c_i32, []),
    "dit_trace_read": (c_i32, [c_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(c_f32)]),
    "dit_status_str": (ctypes.c_char_p, [c_i32]),
    "dit_last_hip_error": (c_i32, []),
}

_lib = None


def load():
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m video_diffusion_transformer_flash_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DitError(RuntimeError):
    pass


def check(status: int, what: str):
    if status != DIT_OK:
        lib = load()
        msg = lib.dit_status_str(status).decode()
        extra = f" (hip error {lib.dit_last_hip_error()})" if status == DIT_EHIP else ""
        raise DitError(f"{what}: {msg}{extra} [{status}]")
