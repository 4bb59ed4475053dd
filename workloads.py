"""Seeded synthetic workloads: shapes, sizes and random inputs, nothing else.

This module is shared by the oracle-side tests, the GPU tests and ``bench.py``.
It holds no step of the method: no paging, no eviction, no attention.  It only
names the workload geometries and draws reproducible inputs for them.

Geometry sources (the pages, cited by title and section):

* p1 = "How the Paged KV Cache Attention Mechanism Enables Long Sequence
  Inference in LingBot-Map", §Implementation Example: 262 tokens per frame made
  of 256 visual patches and 6 special tokens; scale_frames 8, sliding_window 64.
* p2 = "KV Cache Mechanism in LingBot-Map for Streaming Inference: A Deep Dive",
  §Initializing a Model with Custom Cache Settings: patch size 14, so a
  224x224 frame is a 16x16 patch grid and a 518x378 frame a 37x27 grid.
* p3 = "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map",
  §Quantitative Performance Benchmarks: 224x224 frames, 320 frames streamed.
* p2 §Flow-Based Keyframe Selection: keyframes come from a motion threshold;
  here a seeded Bernoulli draw stands in for it (no video, no optical flow).
* p4 = "How LingBot-Map Achieves ~20 FPS Inference with Its KV Cache",
  §Implementation Example: a fixed keyframe interval (4) over a 200-frame
  video; every 4th frame, starting with frame 0, is kept.
* p2 §Configuration Parameters: the cross-frame special switch, here also off
  (nocross_224, otherwise the 224x224 workload).
* One GPU's share when the path is spread over several GPUs: main_224_h2 (2 of
  the 16 heads, a split by head over 8 GPUs) and large_518x378_s1 (one of the
  4 streams, a split by stream over 4 GPUs).
* p3 §Memory Architecture: Paged vs Standard Attention: the full-history
  baseline keeps every frame; noevict_224 is the 224x224 workload with a
  window as long as its 320 frames, so nothing is evicted.

Q/K/V are i.i.d. N(0, 1) (the pages name no dataset; the model and its weights
are not available), rounded to bfloat16 by round-to-nearest-even when the
workload is bf16, so both sides see exactly the same values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    heads: int
    head_dim: int
    dtype: str                 # "bf16" or "fp32"
    tokens_per_frame: int      # T = patches + specials
    num_special: int           # Ns
    special_page: int          # Ps
    scale_frames: int          # S
    sliding_window: int        # W
    frames: int                # frames streamed per stream
    streams: int = 1           # B
    keyframe_p: Optional[float] = None   # Bernoulli keyframe probability
    keyframe_interval: Optional[int] = None   # every k-th frame is a keyframe
    include_scale_frames: bool = True
    cross_frame_special: bool = True
    seed: int = 0
    max_patch_pages: int = 0   # per stream; 0 -> S + W + 1
    max_special_pages: int = 0  # per stream; 0 -> enough for every frame

    @property
    def has_keyframes(self) -> bool:
        """Frames run with eviction deferred, then kept or rolled back."""
        return self.keyframe_p is not None or self.keyframe_interval is not None

    @property
    def patch_page(self) -> int:
        """P = patches per frame: one patch page holds one frame."""
        return self.tokens_per_frame - self.num_special

    @property
    def pmax(self) -> int:
        return self.max_patch_pages or (self.scale_frames + self.sliding_window + 1)

    @property
    def smax(self) -> int:
        if self.max_special_pages:
            return self.max_special_pages
        return -(-(self.frames * self.num_special) // self.special_page)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workload shapes.  Sizes follow the pages' geometry (see header).
TINY = Workload("tiny", layers=1, heads=2, head_dim=64, dtype=FP32,
                tokens_per_frame=22, num_special=6, special_page=8,
                scale_frames=2, sliding_window=4, frames=12)
MAIN = Workload("main_224", layers=1, heads=16, head_dim=64, dtype=BF16,
                tokens_per_frame=262, num_special=6, special_page=16,
                scale_frames=8, sliding_window=64, frames=320)
STACK = MAIN.replace(name="stack_224x24", layers=24)
KEYFRAME = MAIN.replace(name="keyframe_224", frames=1000, keyframe_p=0.3)
INTERVAL = MAIN.replace(name="interval_224", frames=200, keyframe_interval=4)
NOCROSS = MAIN.replace(name="nocross_224", cross_frame_special=False)
# no eviction: the window is as long as the video, so every frame stays
# visible (the full-history contrast)
NOEVICT = MAIN.replace(name="noevict_224", sliding_window=320)
# one GPU's share of the 224x224 workload split by head over 8 GPUs
SHARD_H2 = MAIN.replace(name="main_224_h2", heads=2)
LARGE = Workload("large_518x378", layers=1, heads=16, head_dim=64, dtype=BF16,
                 tokens_per_frame=1005, num_special=6, special_page=16,
                 scale_frames=8, sliding_window=64, frames=200, streams=4)

# one GPU's share of the 518x378 workload split by stream over 4 GPUs
SHARD_S1 = LARGE.replace(name="large_518x378_s1", streams=1)

ALL = {w.name: w for w in (TINY, MAIN, STACK, KEYFRAME, INTERVAL, NOCROSS, NOEVICT,
                           SHARD_H2, LARGE, SHARD_S1)}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite normal draws, so no NaN/Inf handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _frame_seed(seed: int, stream: int, frame: int, layer: int) -> int:
    """A 63-bit seed per (seed, stream, frame, layer) from numpy's SeedSequence."""
    ss = np.random.SeedSequence([seed, stream, frame, layer])
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def frame_qkv_tensors(w: Workload, stream: int, frame: int, layer: int,
                      q_scale: float = 1.0, seed: Optional[int] = None):
    """(q, k, v) torch CPU tensors [T, H, D] in the workload's dtype.

    Drawn with torch's CPU generator (fast enough for the full-size
    workloads); bf16 values come from float32 draws rounded to nearest even.
    ``q_scale`` multiplies q before rounding (a power of two keeps it exact);
    it is used for peaked softmax runs."""
    import torch
    s = w.seed if seed is None else seed
    g = torch.Generator().manual_seed(_frame_seed(s, stream, frame, layer))
    x = torch.randn((3, w.tokens_per_frame, w.heads, w.head_dim),
                    generator=g, dtype=torch.float32)
    if q_scale != 1.0:
        x[0] *= q_scale
    if w.dtype == BF16:
        x = x.to(torch.bfloat16)
    return x[0], x[1], x[2]


def as_numpy(t) -> np.ndarray:
    """torch CPU tensor -> numpy (bfloat16 as uint16 bit patterns)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def frame_qkv(w: Workload, stream: int, frame: int, layer: int,
              q_scale: float = 1.0, seed: Optional[int] = None):
    """(q, k, v) numpy arrays [T, H, D]: bf16 workloads give uint16 bit
    patterns, fp32 workloads float32.  Same values as frame_qkv_tensors."""
    q, k, v = frame_qkv_tensors(w, stream, frame, layer, q_scale, seed)
    return as_numpy(q), as_numpy(k), as_numpy(v)


def keyframe_mask(w: Workload, stream: int = 0) -> np.ndarray:
    """Keyframe flags, one per frame: every keyframe_interval-th frame from
    frame 0, or seeded Bernoulli(keyframe_p) draws.

    All True when the workload has no keyframe selection."""
    if w.keyframe_interval is not None:
        return np.arange(w.frames) % w.keyframe_interval == 0
    if w.keyframe_p is None:
        return np.ones(w.frames, dtype=bool)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0x6B66, stream]))
    return rng.random(w.frames) < w.keyframe_p


def frame_qkv_coded(w: Workload, stream: int, frame: int, layer: int):
    """(q, k, v) torch CPU tensors [T, H, D] (bf16) for token-exact checks.

    q is the usual seeded draw.  Every K row of head h is one vector drawn
    per (seed, layer, head), the same for every token of every frame, so all
    scores of a query row are equal.  Each token's V row is one-hot: the
    token gets a class c in [0, H*D), drawn per (seed, stream, frame, layer,
    row), and V[row, c // D, c % D] = 1, every other element 0.  So the
    token's class is what its V row says, and each (head, dim) column counts
    the visible tokens of that class."""
    import torch
    assert w.dtype == BF16
    T, H, D = w.tokens_per_frame, w.heads, w.head_dim
    q, _, _ = frame_qkv_tensors(w, stream, frame, layer)
    g = torch.Generator().manual_seed(_frame_seed(w.seed, 0x4B, 0, layer))
    key = torch.randn((1, H, D), generator=g, dtype=torch.float32)
    k = key.expand(T, H, D).contiguous().to(torch.bfloat16)
    rng = np.random.default_rng(np.random.SeedSequence(
        [w.seed, 0x5643, stream, frame, layer]))
    cls = rng.integers(0, H * D, size=T)
    v = torch.zeros((T, H * D), dtype=torch.float32)
    v[torch.arange(T), torch.from_numpy(cls)] = 1.0
    return q, k, v.reshape(T, H, D).to(torch.bfloat16)
