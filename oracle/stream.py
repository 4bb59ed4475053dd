"""Streaming driver for the oracle cache (tests and CPU baseline only).

One frame step, for every stream b in order ([p1] §Runtime Flow for Frame
Processing and §Implementation Example: append, then evict, then attention
over the visible pages; [p3] §Visible Page Table Attention: the table is
built once per frame and reused by every layer):

* plain streaming:  begin_frame -> evict;
* keyframe mode ([p2] §Flow-Based Keyframe Selection; [p4] §Deferred
  Eviction and Rollback Mechanism): defer eviction -> begin_frame -> evict
  (recorded as pending);

then the table is built, and for every layer the frame's K/V are written and
its queries attend.  In keyframe mode the frame is afterwards committed
(execute the deferred eviction) when it is a keyframe, or rolled back, and
eviction is re-enabled.

Inputs arrive through a callable, so this package never draws numbers itself.
"""
from __future__ import annotations

from typing import Callable, Iterator, Optional, Sequence

import numpy as np

from .attention import paged_attention
from .cache import OracleCache


def stream_frames(cache: OracleCache,
                  n_frames: int,
                  inputs: Callable[[int, int, int], tuple],
                  keyframes: Optional[Sequence[np.ndarray]] = None,
                  attend: Callable[[int], bool] = lambda t: True,
                  sm_scale: Optional[float] = None,
                  acc=np.float32) -> Iterator[dict]:
    """Run ``n_frames`` lockstep frame steps over every stream of ``cache``.

    ``inputs(b, t, layer) -> (q, k, v)`` gives each [T, H, D].
    ``keyframes[b][t]`` selects keyframe mode (None: plain streaming).
    ``attend(t)`` says whether to compute attention at step t (the page
    bookkeeping and K/V writes always run).

    Yields per step: t, the table, per-layer (o, lse) or None, and per-stream
    stats and free lists taken after the step completed."""
    B = cache.B
    for t in range(n_frames):
        for b in range(B):
            if keyframes is not None:
                cache.set_defer(b, True)
            cache.begin_frame(b)
            cache.evict(b)
        table = cache.build_table()
        outs = []
        for layer in range(cache.L):
            qs = []
            for b in range(B):
                q, k, v = inputs(b, t, layer)
                cache.append_frame(layer, b, k, v)
                qs.append(q)
            if attend(t):
                outs.append(paged_attention(cache.patch_pool[layer],
                                            cache.special_pool[layer], table,
                                            np.concatenate(qs, axis=0),
                                            sm_scale, acc))
            else:
                outs.append(None)
        if keyframes is not None:
            for b in range(B):
                if keyframes[b][t]:
                    cache.execute_deferred_eviction(b)
                else:
                    cache.rollback_last_frame(b)
                cache.set_defer(b, False)
        yield {"t": t, "table": table, "out": outs,
               "stats": [cache.stats(b) for b in range(B)],
               "free": [cache.free_list(b) for b in range(B)]}
