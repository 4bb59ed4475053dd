"""CPU oracle for the paged two-stream KV cache and its prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package; only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path: plain Python lists for the
page bookkeeping and NumPy (float32, and float64 for the brute-force check) for
the arithmetic, written for a reader to check against the pages by eye.

Pages cited (by title; sections named where used):

* [p1] "How the Paged KV Cache Attention Mechanism Enables Long Sequence
  Inference in LingBot-Map"
* [p2] "KV Cache Mechanism in LingBot-Map for Streaming Inference: A Deep Dive"
* [p3] "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map:
  Technical Implementation and Benchmarks"
* [p4] "How LingBot-Map Achieves ~20 FPS Inference with Its KV Cache"

Modules:

* ``pages``       -- one stream's page bookkeeping (free stack, scale pages,
                     sliding window, special counter, defer and rollback).
* ``cache``       -- pools per layer plus a page manager per stream: the
                     ``append_frame`` write, the visible page table, stats.
* ``attention``   -- attention of one frame's queries over the visible pages
                     (gather through the table, two-pass softmax, float32).
* ``brute_force`` -- the same result from the dense frame history and a mask
                     built by frame-index rules (float64), no pages at all.

Every function here is pinned by the ``-m "not gpu"`` tests (worked example of
the stats record, closed forms, invariants, brute force); none is marked
"parity unpinned".
"""
from .pages import (PageError, NoPageError, SpecialFullError, StateError,
                    StreamPages)
from .cache import OracleCache, VisibleTable
from .attention import paged_attention, gather_visible_kv
from .brute_force import BruteForceHistory, dense_masked_attention

__all__ = [
    "PageError", "NoPageError", "SpecialFullError", "StateError",
    "StreamPages", "OracleCache", "VisibleTable", "paged_attention",
    "gather_visible_kv", "BruteForceHistory", "dense_masked_attention",
]
