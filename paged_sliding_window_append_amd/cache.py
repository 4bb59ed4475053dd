"""Thin Python binding over the C ABI: argument marshalling only.

PyTorch supplies device memory (pools, workspace, outputs) and the HIP
stream; every step of the hot path runs in the library's HIP kernels.  There
is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import Config, PageTable, Stats, check

_DT = {"bf16": _lib.PSW_BF16, "fp32": _lib.PSW_FP32}


def _stream_ptr(stream, host_only: bool = False) -> ctypes.c_void_p:
    if host_only and stream is None:
        return ctypes.c_void_p(0)
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_i32)


class Cache:
    """Paged two-stream KV cache of ``streams`` videos over ``layers`` layers.

    ``device=None`` creates the host bookkeeping only (no pools, no
    workspace): page tables, stats and free lists work, device calls raise.
    ``workspace=False`` allocates the pools but binds no workspace: only
    ``append_attention(..., noalloc=True)`` then reaches the device.
    """

    def __init__(self, *, layers: int, streams: int, heads: int, head_dim: int,
                 dtype: str, tokens_per_frame: int, num_special: int,
                 special_page: int, scale_frames: int, sliding_window: int,
                 max_patch_pages: int, max_special_pages: int,
                 max_kv_splits: int = 0, sm_scale: float = 0.0,
                 include_scale_frames: bool = True,
                 cross_frame_special: bool = True,
                 max_frames_per_step: int = 0,
                 device: Optional[str] = "cuda:0", workspace: bool = True):
        self.lib = _lib.load()
        self.cfg = Config(layers, streams, heads, head_dim, _DT[dtype],
                          tokens_per_frame, num_special, special_page,
                          scale_frames, sliding_window, int(include_scale_frames),
                          int(cross_frame_special), max_patch_pages,
                          max_special_pages, max_kv_splits, sm_scale,
                          max_frames_per_step)
        self.dtype = dtype
        self.L, self.B, self.H, self.D = layers, streams, heads, head_dim
        self.T, self.Ns, self.Ps = tokens_per_frame, num_special, special_page
        self.P = tokens_per_frame - num_special
        self.pmax, self.smax = max_patch_pages, max_special_pages
        h = ctypes.c_void_p()
        check(self.lib.psw_create(ctypes.byref(self.cfg), ctypes.byref(h)),
              "psw_create")
        self.h = h
        self.device = device
        self.patch_pools, self.special_pools, self.workspace = [], [], None
        if device is not None:
            self._allocate(device, workspace)

    @classmethod
    def for_workload(cls, w, device: Optional[str] = "cuda:0", **kw):
        return cls(layers=w.layers, streams=w.streams, heads=w.heads,
                   head_dim=w.head_dim, dtype=w.dtype,
                   tokens_per_frame=w.tokens_per_frame,
                   num_special=w.num_special, special_page=w.special_page,
                   scale_frames=w.scale_frames,
                   sliding_window=w.sliding_window, max_patch_pages=w.pmax,
                   max_special_pages=w.smax,
                   include_scale_frames=w.include_scale_frames,
                   cross_frame_special=w.cross_frame_special, device=device, **kw)

    def _allocate(self, device: str, workspace: bool = True) -> None:
        import torch
        pb, sb, wb = (ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t())
        check(self.lib.psw_pool_bytes(ctypes.byref(self.cfg), ctypes.byref(pb),
                                      ctypes.byref(sb), ctypes.byref(wb)),
              "psw_pool_bytes")
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        for layer in range(self.L):
            pp = torch.zeros((self.B * self.pmax, 2, self.P, self.H, self.D),
                             dtype=tdt, device=device)
            sp = torch.zeros((self.B * self.smax, 2, self.Ps, self.H, self.D),
                             dtype=tdt, device=device)
            assert pp.numel() * pp.element_size() == pb.value
            assert sp.numel() * sp.element_size() == sb.value
            check(self.lib.psw_bind_layer(self.h, layer, pp.data_ptr(),
                                          sp.data_ptr()), "psw_bind_layer")
            self.patch_pools.append(pp)
            self.special_pools.append(sp)
        if not workspace:   # for psw_append_attention_noalloc only
            return
        self.workspace = torch.empty(wb.value, dtype=torch.uint8, device=device)
        check(self.lib.psw_bind_workspace(self.h, self.workspace.data_ptr(),
                                          wb.value), "psw_bind_workspace")

    def close(self) -> None:
        if getattr(self, "h", None) is not None and self.h.value:
            self.lib.psw_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- bookkeeping ------------------------------------------------------
    def reset(self, stream: int = -1) -> None:
        check(self.lib.psw_reset(self.h, stream), "psw_reset")

    def begin_frame(self, stream: int) -> None:
        check(self.lib.psw_begin_frame(self.h, stream), "psw_begin_frame")

    def begin_frames(self, stream: int, n: int) -> None:
        """Joint prefill: n frames begun at once, attended together."""
        check(self.lib.psw_begin_frames(self.h, stream, n), "psw_begin_frames")

    def evict_frames(self, stream: int) -> None:
        check(self.lib.psw_evict_frames(self.h, stream), "psw_evict_frames")

    def set_defer_eviction(self, stream: int, on: bool) -> None:
        check(self.lib.psw_set_defer_eviction(self.h, stream, int(bool(on))),
              "psw_set_defer_eviction")

    def execute_deferred_eviction(self, stream: int) -> None:
        check(self.lib.psw_execute_deferred_eviction(self.h, stream),
              "psw_execute_deferred_eviction")

    def rollback_last_frame(self, stream: int) -> None:
        check(self.lib.psw_rollback_last_frame(self.h, stream),
              "psw_rollback_last_frame")

    def stats(self, stream: int) -> dict:
        s = Stats()
        check(self.lib.psw_get_cache_stats(self.h, stream, ctypes.byref(s)),
              "psw_get_cache_stats")
        return s.as_dict()

    def free_list(self, stream: int) -> list:
        n = ctypes.c_int32()
        check(self.lib.psw_export_free_list(self.h, stream, None, 0,
                                            ctypes.byref(n)),
              "psw_export_free_list")
        buf = np.zeros(max(n.value, 1), dtype=np.int32)
        check(self.lib.psw_export_free_list(self.h, stream, _i32p(buf),
                                            n.value, ctypes.byref(n)),
              "psw_export_free_list")
        return buf[:n.value].tolist()

    # ---- table and plan -----------------------------------------------------
    def build_visible_page_table(self) -> dict:
        check(self.lib.psw_build_visible_page_table(self.h),
              "psw_build_visible_page_table")
        return self.page_table()

    def page_table(self) -> dict:
        t = PageTable()
        check(self.lib.psw_get_page_table(self.h, ctypes.byref(t)),
              "psw_get_page_table")
        B = t.num_streams
        arr = lambda p, n: np.ctypeslib.as_array(p, shape=(n,)).copy() if n \
            else np.zeros(0, dtype=np.int32)
        qo = arr(t.qo_indptr, B + 1)
        pind = arr(t.patch_indptr, B + 1)
        sind = arr(t.special_indptr, B + 1)
        return {"qo_indptr": qo, "patch_indptr": pind,
                "patch_ids": arr(t.patch_ids, int(pind[-1])),
                "special_indptr": sind,
                "special_ids": arr(t.special_ids, int(sind[-1])),
                "special_last_len": arr(t.special_last_len, B),
                "special_head_len": arr(t.special_head_len, B),
                "special_tail_first": arr(t.special_tail_first, B),
                "special_tail_len": arr(t.special_tail_len, B)}

    def set_page_table(self, tbl: dict) -> None:
        keep = {k: np.ascontiguousarray(v, dtype=np.int32)
                for k, v in tbl.items()}
        keep["patch_ids"] = keep["patch_ids"] if keep["patch_ids"].size \
            else np.zeros(1, np.int32)
        keep["special_ids"] = keep["special_ids"] if keep["special_ids"].size \
            else np.zeros(1, np.int32)
        seg = [keep[k] if k in keep else None for k in
               ("special_head_len", "special_tail_first", "special_tail_len")]
        t = PageTable(self.B, _i32p(keep["qo_indptr"]),
                      _i32p(keep["patch_indptr"]), _i32p(keep["patch_ids"]),
                      _i32p(keep["special_indptr"]), _i32p(keep["special_ids"]),
                      _i32p(keep["special_last_len"]),
                      *[_i32p(x) if x is not None else None for x in seg])
        check(self.lib.psw_set_page_table(self.h, ctypes.byref(t)),
              "psw_set_page_table")

    def plan(self, stream=None) -> None:
        check(self.lib.psw_plan(self.h, _stream_ptr(stream, self.device is None)),
              "psw_plan")

    def plan_fused(self) -> bool:
        """True when append_attention runs the planned frame as one launch."""
        f = ctypes.c_int32()
        check(self.lib.psw_plan_fused(self.h, ctypes.byref(f)), "psw_plan_fused")
        return bool(f.value)

    def plan_info(self):
        n, s = ctypes.c_int32(), ctypes.c_int32()
        check(self.lib.psw_plan_info(self.h, ctypes.byref(n), ctypes.byref(s)),
              "psw_plan_info")
        return n.value, s.value

    def plan_waves(self) -> int:
        """Waves per workgroup of the planned attention launch (4 or 8)."""
        wv = ctypes.c_int32()
        check(self.lib.psw_plan_waves(self.h, ctypes.byref(wv)), "psw_plan_waves")
        return wv.value

    # ---- device work --------------------------------------------------------
    def _check_rows(self, x, rows: int, name: str) -> None:
        import torch
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if x.dtype != tdt or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {tdt} CUDA tensor")
        if tuple(x.shape) != (rows, self.H, self.D):
            raise ValueError(f"{name} must have shape {(rows, self.H, self.D)}")

    def append_frame(self, layer: int, stream: int, k, v, hip_stream=None):
        """k, v: the stream's current frame [T, H, D] (a chunk of n frames
        begun with begin_frames: [n*T, H, D])."""
        rows = k.shape[0]
        if rows == 0 or rows % self.T:
            raise ValueError(f"k must hold a multiple of T={self.T} rows")
        self._check_rows(k, rows, "k")
        self._check_rows(v, rows, "v")
        check(self.lib.psw_append_frame(self.h, layer, stream, k.data_ptr(),
                                        v.data_ptr(), _stream_ptr(hip_stream)),
              "psw_append_frame")

    def append_frames(self, layer: int, k, v, hip_stream=None):
        rows = k.shape[0]
        self._check_rows(k, rows, "k")
        self._check_rows(v, rows, "v")
        check(self.lib.psw_append_frames(self.h, layer, k.data_ptr(),
                                         v.data_ptr(), _stream_ptr(hip_stream)),
              "psw_append_frames")

    # ---- dense float32 check path (force_fp32) ------------------------------
    def visible_tokens(self) -> np.ndarray:
        """kv_indptr [B+1] of the plan: stream b's dense rows."""
        buf = np.zeros(self.B + 1, dtype=np.int64)
        check(self.lib.psw_visible_tokens(
            self.h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
            "psw_visible_tokens")
        return buf

    def gather_visible_f32(self, layer: int, hip_stream=None):
        """Layer `layer`'s visible K, V of every stream, float [N, H, D]."""
        import torch
        n = int(self.visible_tokens()[-1])
        dev = self.device or "cuda"
        k = torch.empty((max(n, 1), self.H, self.D), dtype=torch.float32, device=dev)
        v = torch.empty_like(k)
        check(self.lib.psw_gather_visible_f32(self.h, layer, k.data_ptr(),
                                              v.data_ptr(), _stream_ptr(hip_stream)),
              "psw_gather_visible_f32")
        return k[:n], v[:n]

    def dense_attention_f32(self, q, k_dense, v_dense, hip_stream=None):
        """Float attention of q over dense rows (as gather_visible_f32)."""
        import torch
        rows = q.shape[0]
        self._check_rows(q, rows, "q")
        n = int(self.visible_tokens()[-1])
        for name, x in (("k_dense", k_dense), ("v_dense", v_dense)):
            if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() \
                    or tuple(x.shape) != (n, self.H, self.D):
                raise ValueError(f"{name} must be a contiguous float32 CUDA "
                                 f"tensor of shape {(n, self.H, self.D)}")
        o = torch.empty((rows, self.H, self.D), dtype=torch.float32, device=q.device)
        lse = torch.empty((rows, self.H), dtype=torch.float32, device=q.device)
        check(self.lib.psw_dense_attention_f32(
            self.h, q.data_ptr(), k_dense.data_ptr(), v_dense.data_ptr(),
            o.data_ptr(), lse.data_ptr(), _stream_ptr(hip_stream)),
            "psw_dense_attention_f32")
        return o, lse

    def attention(self, layer: int, q, o=None, lse=None, hip_stream=None):
        import torch
        rows = q.shape[0]
        self._check_rows(q, rows, "q")
        if o is None:
            o = torch.empty_like(q)
        self._check_rows(o, rows, "o")
        if lse is None:
            lse = torch.empty((rows, self.H), dtype=torch.float32,
                              device=q.device)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (rows, self.H) \
                or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [rows, H]")
        check(self.lib.psw_attention(self.h, layer, q.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), _stream_ptr(hip_stream)),
              "psw_attention")
        return o, lse

    def append_attention(self, layer: int, k, v, q, o=None, lse=None,
                         hip_stream=None, noalloc: bool = False):
        """append_frames(layer, k, v) then attention(layer, q): one launch
        when the plan fits the kernel arguments.  ``noalloc``: through
        psw_append_attention_noalloc (the library's scratch array instead of
        the bound workspace; pass o and lse to allocate nothing here either)."""
        import torch
        rows = q.shape[0]
        self._check_rows(k, k.shape[0], "k")
        self._check_rows(v, k.shape[0], "v")
        self._check_rows(q, rows, "q")
        if o is None:
            o = torch.empty_like(q)
        self._check_rows(o, rows, "o")
        if lse is None:
            lse = torch.empty((rows, self.H), dtype=torch.float32,
                              device=q.device)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (rows, self.H) \
                or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [rows, H]")
        fn, name = (self.lib.psw_append_attention_noalloc, "psw_append_attention_noalloc") \
            if noalloc else (self.lib.psw_append_attention, "psw_append_attention")
        check(fn(self.h, layer, k.data_ptr(), v.data_ptr(), q.data_ptr(),
                 o.data_ptr(), lse.data_ptr(), _stream_ptr(hip_stream)), name)
        return o, lse
