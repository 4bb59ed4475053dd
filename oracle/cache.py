"""Paged two-stream KV cache over B streams and L layers (oracle, tests only).

The pools follow the physical layout the pages give for the page store, a
5-D array ``[pages, 2, page_size, H, D]`` ([p1] §Physical Memory Layout).
That section reads the axis of size 2 as the two streams, which cannot hold
patch pages and special pages of different sizes; the reading taken here is
one pool per page stream, with the axis of size 2 holding K (0) and V (1).

Streams share one pool per layer: stream b owns patch pages
[b*pmax, (b+1)*pmax) and special pages [b*smax, (b+1)*smax), so one table in
CSR form can list the pages of all streams at once.

``append_frame`` splits the frame's K/V rows between the two page streams
([p1] §Appending New Frames).  Reading: rows [0, Ns) of a frame are its
special tokens and rows [Ns, T) its patches.

``build_table`` forms the visible page table: scale pages and the most
recent window pages of the patch stream, every special page written so far,
and the number of valid tokens in the last special page ([p1] §Building the
Visible Page Table; [p1] FAQ on variable token counts).  It is built once
per frame and used by every layer ([p3] §Visible Page Table Attention).
Without cross-frame specials ([p2] §Configuration Parameters) the visible
specials are a head range (the scale frames') and a tail range (the visible
window frames'), so the table also carries, per stream, the head length and
where the tail starts and ends: the listed special pages are the head's
pages, then the tail's pages.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from .pages import StateError, StreamPages


@dataclasses.dataclass
class VisibleTable:
    """Visible pages of every stream, CSR over streams (int32 arrays)."""
    qo_indptr: np.ndarray        # [B+1] query rows of each stream
    patch_indptr: np.ndarray     # [B+1]
    patch_ids: np.ndarray        # global patch page IDs, table order
    special_indptr: np.ndarray   # [B+1]
    special_ids: np.ndarray      # global special page IDs
    special_last_len: np.ndarray  # [B] valid tokens in the last special page
    # Visible specials of stream b: the first special_head_len[b] tokens of
    # the listed pages (from slot 0 of the first), then special_tail_len[b]
    # tokens from slot special_tail_first[b] of the page after the head's.
    special_head_len: np.ndarray    # [B]
    special_tail_first: np.ndarray  # [B]
    special_tail_len: np.ndarray    # [B]

    def kv_len(self, b: int, P: int, Ps: int) -> int:
        npatch = int(self.patch_indptr[b + 1] - self.patch_indptr[b])
        return (npatch * P + int(self.special_head_len[b]) +
                int(self.special_tail_len[b]))


class OracleCache:
    def __init__(self, *, layers: int, streams: int, heads: int, head_dim: int,
                 tokens_per_frame: int, num_special: int, special_page: int,
                 scale_frames: int, sliding_window: int, pmax: int, smax: int,
                 storage=np.uint16, include_scale_frames: bool = True,
                 cross_frame_special: bool = True):
        self.L, self.B, self.H, self.D = layers, streams, heads, head_dim
        self.T, self.Ns, self.Ps = tokens_per_frame, num_special, special_page
        self.P = tokens_per_frame - num_special
        if self.P < 1:
            raise ValueError("a frame needs at least one patch token")
        self.pmax, self.smax = pmax, smax
        self.streams: List[StreamPages] = [
            StreamPages(scale_frames, sliding_window, num_special,
                        special_page, pmax, smax, include_scale_frames,
                        cross_frame_special) for _ in range(streams)]
        self.patch_pool = [np.zeros((streams * pmax, 2, self.P, heads, head_dim),
                                    dtype=storage) for _ in range(layers)]
        self.special_pool = [np.zeros((streams * smax, 2, special_page, heads,
                                       head_dim), dtype=storage)
                             for _ in range(layers)]

    @classmethod
    def for_workload(cls, w, storage=None):
        if storage is None:
            storage = np.uint16 if w.dtype == "bf16" else np.float32
        return cls(layers=w.layers, streams=w.streams, heads=w.heads,
                   head_dim=w.head_dim, tokens_per_frame=w.tokens_per_frame,
                   num_special=w.num_special, special_page=w.special_page,
                   scale_frames=w.scale_frames, sliding_window=w.sliding_window,
                   pmax=w.pmax, smax=w.smax, storage=storage,
                   include_scale_frames=w.include_scale_frames,
                   cross_frame_special=w.cross_frame_special)

    # -- bookkeeping, per stream ---------------------------------------------
    def reset(self, b: int = -1) -> None:
        """Clear one stream (or all): the cache reset between videos."""
        for i, s in enumerate(self.streams):
            if b < 0 or b == i:
                s.reset()

    def begin_frame(self, b: int):
        return self.streams[b].begin_frame()

    def begin_frames(self, b: int, n: int):
        """Joint prefill: n frames of stream b begun as one chunk."""
        return self.streams[b].begin_frames(n)

    def evict(self, b: int) -> int:
        return self.streams[b].evict()

    def set_defer(self, b: int, on: bool) -> None:
        self.streams[b].set_defer(on)

    def execute_deferred_eviction(self, b: int) -> int:
        return self.streams[b].execute_deferred_eviction()

    def rollback_last_frame(self, b: int) -> None:
        self.streams[b].rollback_last_frame()

    def stats(self, b: int) -> dict:
        return self.streams[b].stats()

    def free_list(self, b: int) -> List[int]:
        """Free stack of stream b, bottom first, as global page IDs."""
        return [b * self.pmax + p for p in self.streams[b].free]

    # -- the K/V write of append_frame -------------------------------------
    def append_frame(self, layer: int, b: int, k: np.ndarray, v: np.ndarray):
        """Write the current frame's K and V ([T, H, D] each; a chunk of n
        frames: [n*T, H, D], frame after frame) into layer's pools."""
        frames = self.streams[b].current_frames()
        n = len(frames)
        if k.shape != (n * self.T, self.H, self.D) or v.shape != k.shape:
            raise ValueError("k and v must be [n*T, H, D]")
        pp = self.patch_pool[layer]
        sp = self.special_pool[layer]
        for f, (page, positions) in enumerate(frames):
            kf, vf = k[f * self.T:(f + 1) * self.T], v[f * self.T:(f + 1) * self.T]
            gpage = b * self.pmax + page
            # patches: rows Ns..T-1 fill slots 0..P-1 of the frame's patch page
            pp[gpage, 0] = kf[self.Ns:]
            pp[gpage, 1] = vf[self.Ns:]
            # specials: row r goes to the stream's special position positions[r]
            for r, pos in enumerate(positions):
                spage = b * self.smax + pos // self.Ps
                slot = pos % self.Ps
                sp[spage, 0, slot] = kf[r]
                sp[spage, 1, slot] = vf[r]

    # -- the visible page table ----------------------------------------------
    def build_table(self) -> VisibleTable:
        """Table over all streams.  A stream takes part when it has a current
        frame (begun and not rolled back): its queries attend, T rows per
        frame of the last begin.  Other streams get empty ranges."""
        qo, pind, sind, pids, sids, last = [0], [0], [0], [], [], []
        head, tfirst, tlen = [], [], []
        Ps = self.Ps
        for b, s in enumerate(self.streams):
            if s.cur is None:
                qo.append(qo[-1])
                pind.append(pind[-1])
                sind.append(sind[-1])
                last.append(0)
                head.append(0)
                tfirst.append(0)
                tlen.append(0)
                continue
            vp = s.visible_patch_pages()
            pids += [b * self.pmax + p for p in vp]
            segs = s.visible_special_segments()
            # head: a range starting at position 0 (possibly empty); tail:
            # the range after it, if any
            if segs and segs[0][0] == 0:
                h_len, rest = segs[0][1], segs[1:]
            else:
                h_len, rest = 0, segs
            t_start, t_end = rest[0] if rest else (0, 0)
            pages = list(range(-(-h_len // Ps)))
            if t_end > t_start:
                pages += list(range(t_start // Ps, -(-t_end // Ps)))
            sids += [b * self.smax + p for p in pages]
            end = t_end if t_end > t_start else h_len
            last.append(end - (-(-end // Ps) - 1) * Ps if end > 0 else 0)
            head.append(h_len)
            tfirst.append(t_start % Ps if t_end > t_start else 0)
            tlen.append(t_end - t_start)
            qo.append(qo[-1] + len(s.cur) * self.T)
            pind.append(len(pids))
            sind.append(len(sids))
        i32 = lambda x: np.asarray(x, dtype=np.int32)
        return VisibleTable(i32(qo), i32(pind), i32(pids), i32(sind), i32(sids),
                            i32(last), i32(head), i32(tfirst), i32(tlen))

    def require_frame(self, b: int) -> None:
        if self.streams[b].frame_count == 0:
            raise StateError("stream has no frame")
