"""One stream's page bookkeeping, in plain Python lists (oracle, tests only).

What the pages fix:

* Patch stream: one patch page per frame, sized to the frame's patch count;
  pages leave through eviction onto a free list and are reused for later
  frames ([p1] §Patch Stream (Recyclable); [p3] §Constant Memory with
  Two-Stream Paging).
* The first ``scale_frames`` frames stay resident for good; the most recent
  frames are kept up to ``sliding_window`` ([p2] §Patch Stream (Recyclable)).
* Eviction: while the live window pages exceed the window, the oldest window
  page goes back to the free list; scale pages and special pages are never
  touched ([p2] §Sliding-Window Eviction Strategy, steps 1-3; [p1] §Evicting
  Stale Frames).
* Special stream: the special tokens of each frame are packed one after the
  other into append-only pages that are never evicted ([p1] §Special Stream
  (Append-Only); [p2] §Special Stream (Append-Only)).
* Deferred eviction, then commit (execute the deferred eviction) or undo the
  last frame ([p2] §Flow-Based Keyframe Selection; [p4] §Deferred Eviction
  and Rollback Mechanism).
* Statistics record with frame_count, scale_pages, live_pages, free_pages,
  special_tokens ([p3] §Monitoring Cache Statistics).
* Two switches ([p2] §Configuration Parameters): whether special tokens of
  evicted frames stay available to later frames (cross-frame specials, the
  default) and whether scale frames are kept at all (the default).

Joint prefill ([p2] §Sliding-Window Eviction Strategy and the FAQ on
disabling the window: the scale frames keep a bidirectional context): n
frames may be begun at once as one chunk, which is n single-frame allocations
in a row whose queries then attend together; a rollback undoes the whole
chunk, and a chunk of more than one frame may put at most W frames into the
window (an eviction would otherwise take a page of the chunk).

Readings taken where the pages are silent (each also listed in the design
notes): the free list is a LIFO stack whose first pops are 0, 1, 2, ...; the
scale frames are the first kept frames; eviction runs before attention, so the
window count includes the current frame; while an eviction is deferred the
visible window is still the last ``sliding_window`` window pages; a rollback
returns the frame's page to the top of the free stack and gives back its
special slots; a non-deferred eviction that removed a page ends the undo
window (the frame can no longer be rolled back exactly).  Without scale
frames every frame is a window frame (scale_frames acts as 0).  Without
cross-frame specials the visible special tokens are exactly those of the
frames whose patch pages are visible; the special pages themselves stay
append-only (they are never recycled either way).
"""
from __future__ import annotations

from typing import List, Optional, Tuple


class PageError(RuntimeError):
    code = -1


class NoPageError(PageError):
    """The patch free list is empty."""
    code = -2


class SpecialFullError(PageError):
    """The special pool cannot take another frame's special tokens."""
    code = -3


class StateError(PageError):
    """The call is not valid in the current state (e.g. nothing to undo)."""
    code = -4


class StreamPages:
    """Bookkeeping of one video stream (both page streams).

    Page IDs are local to the stream (0 .. pmax-1 patch, 0 .. smax-1 special);
    ``OracleCache`` adds the stream's base when it forms a shared table.
    """

    def __init__(self, scale_frames: int, sliding_window: int,
                 num_special: int, special_page: int,
                 pmax: int, smax: int, include_scale_frames: bool = True,
                 cross_frame_special: bool = True):
        if scale_frames < 0 or sliding_window < 0:
            raise PageError("scale_frames and sliding_window must be >= 0")
        if not include_scale_frames:
            scale_frames = 0
        if scale_frames == 0 and sliding_window == 0 and not cross_frame_special:
            raise PageError("nothing would ever be visible")
        if num_special < 1 or special_page < 1:
            raise PageError("need at least one special token and slot")
        if pmax < scale_frames + sliding_window + 1:
            raise PageError("patch pool must hold scale + window + 1 pages")
        if smax < 1:
            raise PageError("special pool needs at least one page")
        self.S = scale_frames
        self.W = sliding_window
        self.Ns = num_special
        self.Ps = special_page
        self.pmax = pmax
        self.smax = smax
        self.cross_frame_special = bool(cross_frame_special)
        self.reset()

    # -- state -----------------------------------------------------------
    def reset(self) -> None:
        """Empty cache: every patch page on the free stack, no specials."""
        # Stack top is the list end, so pops yield 0, 1, 2, ... first.
        self.free: List[int] = list(range(self.pmax - 1, -1, -1))
        self.scale: List[int] = []
        self.window: List[int] = []      # oldest first
        self.n_special = 0               # special tokens written so far
        self.frame_count = 0
        self.defer = False
        self.pending = False             # an eviction was deferred
        # per frame of the last begin: (page, "scale"|"window")
        self.undo: Optional[List[Tuple[int, str]]] = None
        # Where the most recent begin put its frames, (page, special
        # positions) per frame; the K/V write of every layer goes there.
        # Cleared by rollback and reset.
        self.cur: Optional[List[Tuple[int, List[int]]]] = None

    def state(self):
        """The part of the state a rollback must restore exactly."""
        return (tuple(self.free), tuple(self.scale), tuple(self.window),
                self.n_special, self.frame_count)

    # -- append_frame (bookkeeping half) --------------------------------
    def begin_frame(self) -> Tuple[int, List[int]]:
        """Allocate the new frame: one patch page and Ns special positions.

        Returns (patch page, special token positions).  Fails without
        changing anything when a pool is exhausted."""
        return self.begin_frames(1)[0]

    def begin_frames(self, n: int) -> List[Tuple[int, List[int]]]:
        """Allocate n frames at once (a joint-prefill chunk): n single-frame
        allocations in a row.  Returns (page, positions) per frame."""
        if n < 1:
            raise PageError("a chunk has at least one frame")
        to_scale = min(n, self.S - len(self.scale))
        if n > 1 and n - to_scale > self.W:
            raise PageError("more chunk frames for the window than it keeps")
        if len(self.free) < n:
            raise NoPageError("no free patch page")
        if self.n_special + n * self.Ns > self.smax * self.Ps:
            raise SpecialFullError("special pool full")
        frames, undo = [], []
        for _ in range(n):
            page = self.free.pop()
            if len(self.scale) < self.S:
                self.scale.append(page)
                undo.append((page, "scale"))
            else:
                self.window.append(page)
                undo.append((page, "window"))
            frames.append((page, list(range(self.n_special,
                                            self.n_special + self.Ns))))
            self.n_special += self.Ns
            self.frame_count += 1
        self.undo = undo
        self.cur = frames
        return frames

    def current_frames(self) -> List[Tuple[int, List[int]]]:
        """(patch page, special positions) of each frame of the last begin."""
        if self.cur is None:
            raise StateError("no begun frame to write")
        return self.cur

    # -- eviction ----------------------------------------------------------
    def _evict_now(self) -> int:
        evicted = 0
        while len(self.window) > self.W:
            self.free.append(self.window.pop(0))
            evicted += 1
        self.pending = False
        if evicted:
            self.undo = None
        return evicted

    def evict(self) -> int:
        """Sliding-window eviction; recorded as pending while deferred."""
        if self.defer:
            self.pending = len(self.window) > self.W
            return 0
        return self._evict_now()

    def set_defer(self, on: bool) -> None:
        self.defer = bool(on)

    def execute_deferred_eviction(self) -> int:
        """Commit: run the eviction now, whatever the defer flag says."""
        return self._evict_now()

    def rollback_last_frame(self) -> None:
        """Exact inverse of the last ``begin_frame`` or ``begin_frames`` (if
        nothing was evicted since): its pages return to the free stack, its
        specials are released and the frame count goes back."""
        if self.undo is None:
            raise StateError("no frame to roll back")
        for page, where in reversed(self.undo):
            lst = self.scale if where == "scale" else self.window
            assert lst and lst[-1] == page
            lst.pop()
            self.free.append(page)
            self.n_special -= self.Ns
            self.frame_count -= 1
        self.pending = False
        self.undo = None
        self.cur = None

    # -- visible table -----------------------------------------------------
    def visible_patch_pages(self) -> List[int]:
        """Scale pages, then the most recent W window pages (oldest first)."""
        start = max(0, len(self.window) - self.W)
        win = self.window[start:]
        return list(self.scale) + list(win)

    def visible_special_pages(self) -> Tuple[List[int], int]:
        """All special pages written so far and the fill of the last one."""
        if self.n_special == 0:
            return [], 0
        npages = -(-self.n_special // self.Ps)
        last = self.n_special - (npages - 1) * self.Ps
        return list(range(npages)), last

    def visible_special_segments(self) -> List[Tuple[int, int]]:
        """Visible special-token positions as [start, end) ranges.

        Kept frame f (0-based, in keep order) owns positions
        [f*Ns, (f+1)*Ns).  With cross-frame specials every kept frame's
        tokens are visible: one range [0, n).  Without, only the frames whose
        patch pages are visible: the scale frames (a prefix) and the last
        visible window frames (a suffix), so at most two ranges."""
        n = self.n_special
        if n == 0:
            return []
        if self.cross_frame_special:
            return [(0, n)]
        head = len(self.scale) * self.Ns
        visible_window = min(self.W, len(self.window))
        tail = (self.frame_count - visible_window) * self.Ns   # >= head
        if tail == head:
            return [(0, n)]
        segs = [(0, head)] if head > 0 else []
        if tail < n:
            segs.append((tail, n))
        return segs

    def stats(self) -> dict:
        return {"frame_count": self.frame_count,
                "scale_pages": len(self.scale),
                "live_pages": len(self.window),
                "free_pages": len(self.free),
                "special_tokens": self.n_special}
