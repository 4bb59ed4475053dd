"""Dense masked attention over the whole frame history (oracle, tests only).

No pages, no free list, no table: every frame ever processed is kept in a
dense history, and the keys visible to the current frame are chosen by
frame-index rules taken straight from the pages' description of what stays
resident:

* (i)   the patch tokens of the first ``scale_frames`` kept frames
        ([p2] §Patch Stream (Recyclable), scale pages);
* (ii)  the patch tokens of the last ``sliding_window`` kept frames that are
        not scale frames ([p2] §Patch Stream (Recyclable), sliding window;
        [p2] §Sliding-Window Eviction Strategy);
* (iii) the special tokens of every kept frame, evicted or not
        ([p1] §Special Stream (Append-Only); cross-frame special retention,
        [p2] §Configuration Parameters).

The two switches of [p2] §Configuration Parameters: without cross-frame
specials, (iii) shrinks to the frames of (i) and (ii); without scale frames,
(i) is empty and (ii) takes the last ``sliding_window`` kept frames.

"Kept" frames are the ones committed to the cache; a rolled-back frame is not
kept ([p2] §Flow-Based Keyframe Selection).  The current frame is resident
while it is processed, whether or not it is kept afterwards.  A joint-prefill
chunk of n frames is current as a whole: all n are resident, and the queries
of every one of them see the same keys.  Reading: rows
[0, Ns) of each frame are its special tokens.

Everything is float64; the result is the plain definition the paged path has
to reproduce.
"""
from __future__ import annotations

from typing import List

import numpy as np


def _to_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:   # bfloat16 bit patterns
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float64)


def dense_masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           mask: np.ndarray, sm_scale: float):
    """q [Tq, H, D] over k, v [N, H, D] with a boolean key mask [N].

    Masked keys get a score of minus infinity.  Returns (o, lse) float64."""
    q, k, v = _to_f64(q), _to_f64(k), _to_f64(v)
    Tq, H, D = q.shape
    o = np.zeros((Tq, H, D))
    lse = np.zeros((Tq, H))
    for h in range(H):
        s = (q[:, h] @ k[:, h].T) * sm_scale
        s = np.where(mask[None, :], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        o[:, h] = (w @ v[:, h]) / l
        lse[:, h] = (m + np.log(l))[:, 0]
    return o, lse


class BruteForceHistory:
    """Dense history of one stream's frames and which of them were kept."""

    def __init__(self, num_special: int, scale_frames: int,
                 sliding_window: int, include_scale_frames: bool = True,
                 cross_frame_special: bool = True):
        self.Ns = num_special
        self.S = scale_frames if include_scale_frames else 0
        self.W = sliding_window
        self.cross_frame_special = cross_frame_special
        self.k: List[np.ndarray] = []
        self.v: List[np.ndarray] = []
        self.kept: List[bool] = []
        self.n_cur = 0          # frames of the current chunk (the last ones)

    def push(self, k: np.ndarray, v: np.ndarray) -> None:
        """A new current frame (resident while processed)."""
        self.push_chunk([k], [v])

    def push_chunk(self, ks: List[np.ndarray], vs: List[np.ndarray]) -> None:
        """A joint-prefill chunk of frames, current together."""
        self.k += list(ks)
        self.v += list(vs)
        self.kept += [True] * len(ks)
        self.n_cur = len(ks)

    def drop_current(self) -> None:
        """The current frame (or chunk) is not kept (rolled back)."""
        for f in range(len(self.k) - self.n_cur, len(self.k)):
            self.kept[f] = False

    def resident_frames(self) -> List[int]:
        """Kept frames before the current chunk, then the chunk's frames."""
        c = len(self.k) - self.n_cur
        return [f for f in range(c) if self.kept[f]] + list(range(c, len(self.k)))

    def visible_mask(self) -> np.ndarray:
        """Boolean mask over the concatenated history [frames * T]."""
        T = self.k[0].shape[0]
        R = self.resident_frames()
        scale = R[:self.S]
        rest = R[self.S:]
        window = rest[max(0, len(rest) - self.W):] if self.W > 0 else []
        mask = np.zeros(len(self.k) * T, dtype=bool)
        for f in (R if self.cross_frame_special else scale + window):   # (iii)
            mask[f * T: f * T + self.Ns] = True
        for f in scale + window:             # (i) and (ii) patches
            mask[f * T + self.Ns: (f + 1) * T] = True
        return mask

    def attend(self, q: np.ndarray, sm_scale: float | None = None):
        """Attention of the current frame's queries q [T, H, D] (a chunk's:
        [n*T, H, D], all with the same visible keys)."""
        if sm_scale is None:
            sm_scale = 1.0 / np.sqrt(q.shape[2])
        k = np.concatenate(self.k, axis=0)
        v = np.concatenate(self.v, axis=0)
        return dense_masked_attention(q, k, v, self.visible_mask(), sm_scale)

    def visible_count(self) -> int:
        return int(self.visible_mask().sum())
