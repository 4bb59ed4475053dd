"""ctypes declarations of the C ABI in include/psw.h (argument marshalling
only).  Loading fails loudly when libpsw.so has not been built."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpsw.so")

PSW_OK = 0
STATUS_NAMES = {0: "PSW_OK", -1: "PSW_EINVAL", -2: "PSW_ENOPAGE",
                -3: "PSW_ESPECIAL_FULL", -4: "PSW_ESTATE", -5: "PSW_EHIP",
                -6: "PSW_EUNBOUND"}
PSW_BF16, PSW_FP32 = 0, 1

i32 = ctypes.c_int32
P_i32 = ctypes.POINTER(ctypes.c_int32)
vp = ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("num_layers", i32), ("num_streams", i32),
                ("num_heads", i32), ("head_dim", i32), ("dtype", i32),
                ("tokens_per_frame", i32), ("num_special_tokens", i32),
                ("special_page_size", i32), ("scale_frames", i32),
                ("sliding_window", i32), ("include_scale_frames", i32),
                ("cross_frame_special", i32), ("max_patch_pages", i32),
                ("max_special_pages", i32), ("max_kv_splits", i32),
                ("sm_scale", ctypes.c_float), ("max_frames_per_step", i32)]


class Stats(ctypes.Structure):
    _fields_ = [("frame_count", i32), ("scale_pages", i32),
                ("live_pages", i32), ("free_pages", i32),
                ("special_tokens", i32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PageTable(ctypes.Structure):
    _fields_ = [("num_streams", i32), ("qo_indptr", P_i32),
                ("patch_indptr", P_i32), ("patch_ids", P_i32),
                ("special_indptr", P_i32), ("special_ids", P_i32),
                ("special_last_len", P_i32), ("special_head_len", P_i32),
                ("special_tail_first", P_i32), ("special_tail_len", P_i32)]


# name -> (restype, argtypes)
SIGNATURES = {
    "psw_last_error": (ctypes.c_char_p, []),
    "psw_config_check": (i32, [ctypes.POINTER(Config)]),
    "psw_pool_bytes": (i32, [ctypes.POINTER(Config),
                             ctypes.POINTER(ctypes.c_size_t),
                             ctypes.POINTER(ctypes.c_size_t),
                             ctypes.POINTER(ctypes.c_size_t)]),
    "psw_create": (i32, [ctypes.POINTER(Config), ctypes.POINTER(vp)]),
    "psw_destroy": (None, [vp]),
    "psw_bind_layer": (i32, [vp, i32, vp, vp]),
    "psw_bind_workspace": (i32, [vp, vp, ctypes.c_size_t]),
    "psw_reset": (i32, [vp, i32]),
    "psw_begin_frame": (i32, [vp, i32]),
    "psw_begin_frames": (i32, [vp, i32, i32]),
    "psw_evict_frames": (i32, [vp, i32]),
    "psw_set_defer_eviction": (i32, [vp, i32, i32]),
    "psw_execute_deferred_eviction": (i32, [vp, i32]),
    "psw_rollback_last_frame": (i32, [vp, i32]),
    "psw_append_frame": (i32, [vp, i32, i32, vp, vp, vp]),
    "psw_append_frames": (i32, [vp, i32, vp, vp, vp]),
    "psw_build_visible_page_table": (i32, [vp]),
    "psw_get_page_table": (i32, [vp, ctypes.POINTER(PageTable)]),
    "psw_set_page_table": (i32, [vp, ctypes.POINTER(PageTable)]),
    "psw_plan": (i32, [vp, vp]),
    "psw_attention": (i32, [vp, i32, vp, vp, vp, vp]),
    "psw_append_attention": (i32, [vp, i32, vp, vp, vp, vp, vp, vp]),
    "psw_append_attention_noalloc": (i32, [vp, i32, vp, vp, vp, vp, vp, vp]),
    "psw_plan_fused": (i32, [vp, P_i32]),
    "psw_visible_tokens": (i32, [vp, ctypes.POINTER(ctypes.c_int64)]),
    "psw_gather_visible_f32": (i32, [vp, i32, vp, vp, vp]),
    "psw_dense_attention_f32": (i32, [vp, vp, vp, vp, vp, vp, vp]),
    "psw_get_cache_stats": (i32, [vp, i32, ctypes.POINTER(Stats)]),
    "psw_export_free_list": (i32, [vp, i32, P_i32, i32, P_i32]),
    "psw_plan_info": (i32, [vp, P_i32, P_i32]),
    "psw_plan_waves": (i32, [vp, P_i32]),
    "psw_profile_enable": (i32, [vp, i32]),
    "psw_profile_read": (i32, [vp, ctypes.POINTER(ctypes.c_double), P_i32,
                               ctypes.POINTER(ctypes.c_double), P_i32]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m paged_sliding_window_append_amd.build`")
    # torch first: its HIP runtime has the soname libpsw.so asks for, so the
    # library binds to the runtime that owns the caller's streams and device
    # memory.  Loaded the other way round, the process maps two HIP runtimes
    # and the library's device queries fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PswError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def check(status: int, where: str) -> None:
    if status != PSW_OK:
        msg = load().psw_last_error()
        raise PswError(status, where, msg.decode() if msg else "")
