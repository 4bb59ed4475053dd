"""Pins for the oracle's page bookkeeping (CPU only).

Each test checks the oracle against something other than itself: the pages'
printed stats record, closed forms of the table sizes, invariants the pages
state (specials never evicted, window bounded, freed pages reused, exact
last-page length, rollback restores the previous state) and counts the pages
print for keyframe selection.
"""
import json
import os
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import NoPageError, StateError, StreamPages
from oracle.cache import OracleCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_stats_worked_example():
    g = _golden("stats_worked_example.json")
    c = g["config"]
    s = StreamPages(c["scale_frames"], c["sliding_window"], c["num_special"],
                    c["special_page"], c["max_patch_pages"], 64)
    for _ in range(c["frames"]):
        s.begin_frame()
        s.evict()
    assert s.stats() == g["expected"]


def test_fixed_interval_keyframes_count():
    """Every 4th of 200 frames kept: the non-keyframes are processed with
    eviction deferred and then removed again."""
    g = _golden("fixed_interval.json")
    c = g["config"]
    s = StreamPages(c["scale_frames"], c["sliding_window"], c["num_special"],
                    c["special_page"], c["scale_frames"] + c["sliding_window"] + 1,
                    64)
    for t in range(c["frames"]):
        s.set_defer(True)
        s.begin_frame()
        s.evict()
        if t % c["keyframe_interval"] == 0:
            s.execute_deferred_eviction()
        else:
            s.rollback_last_frame()
        s.set_defer(False)
    st_ = s.stats()
    assert st_["frame_count"] == g["expected"]["kept_frames"]
    assert st_["special_tokens"] == g["expected"]["special_tokens"]


@pytest.mark.parametrize("T,Ns,Ps,S,W,frames", [
    (22, 6, 8, 2, 4, 12),      # tiny workload
    (262, 6, 16, 8, 64, 320),  # 224x224 workload
    (1005, 6, 16, 8, 64, 200),  # 518x378 workload
    (10, 3, 5, 0, 3, 20),
    (10, 3, 7, 3, 0, 20),      # no sliding window at all
])
def test_table_closed_forms(T, Ns, Ps, S, W, frames):
    """Visible token count, special page count and last-page fill per frame:
    Lkv(t) = P*min(t+1, S+W) + Ns*(t+1); ceil(Ns(t+1)/Ps) special pages;
    last page holds ((Ns(t+1)-1) mod Ps) + 1 tokens."""
    P = T - Ns
    cache = OracleCache(layers=1, streams=1, heads=1, head_dim=1,
                        tokens_per_frame=T, num_special=Ns, special_page=Ps,
                        scale_frames=S, sliding_window=W, pmax=S + W + 1,
                        smax=-(-frames * Ns // Ps))
    for t in range(frames):
        cache.begin_frame(0)
        cache.evict(0)
        tb = cache.build_table()
        n = Ns * (t + 1)
        assert tb.kv_len(0, P, Ps) == P * min(t + 1, S + W) + n
        assert len(tb.special_ids) == -(-n // Ps)
        assert tb.special_last_len[0] == (n - 1) % Ps + 1
        assert list(tb.qo_indptr) == [0, T]


def test_tiny_last_page_cycle():
    """Tiny workload: six specials per frame into pages of 8 slots gives the
    last-page fill cycle 6, 4, 2, 8 and 22, 44, ..., 132, 138, ..., 168
    visible tokens."""
    cache = OracleCache(layers=1, streams=1, heads=1, head_dim=1,
                        tokens_per_frame=22, num_special=6, special_page=8,
                        scale_frames=2, sliding_window=4, pmax=7, smax=9)
    lpl, lkv = [], []
    for _ in range(12):
        cache.begin_frame(0)
        cache.evict(0)
        tb = cache.build_table()
        lpl.append(int(tb.special_last_len[0]))
        lkv.append(tb.kv_len(0, 16, 8))
    assert lpl == [6, 4, 2, 8] * 3
    assert lkv == [22, 44, 66, 88, 110, 132, 138, 144, 150, 156, 162, 168]


def test_steady_state_visible_pages_main():
    """8 scale + 64 window = 72 visible patch pages once the window is full
    (the pages' "~70" visible pages for a 64-frame window)."""
    s = StreamPages(8, 64, 6, 16, 73, 120)
    counts = []
    for t in range(320):
        s.begin_frame()
        s.evict()
        counts.append(len(s.visible_patch_pages()))
    assert counts[70] == 71 and all(c == 72 for c in counts[71:])
    assert s.stats()["special_tokens"] == 320 * 6


def test_lifo_reuse_plain_streaming():
    """Once the window is full the page evicted at step t is the page the
    next frame gets (free list reused, top of stack first)."""
    s = StreamPages(2, 3, 1, 4, 6, 64)
    evicted_prev = None
    for t in range(40):
        page, _ = s.begin_frame()
        if evicted_prev is not None:
            assert page == evicted_prev
        before = list(s.window)
        s.evict()
        gone = [p for p in before if p not in s.window]
        evicted_prev = gone[0] if gone else None
        if t >= 5:
            assert len(gone) == 1


def test_error_paths_strong_guarantee():
    s = StreamPages(1, 1, 2, 4, 3, 2)
    with pytest.raises(StateError):
        s.rollback_last_frame()
    s.begin_frame(); s.evict()
    s.begin_frame(); s.evict()
    s.set_defer(True)
    s.begin_frame(); s.evict()          # pool now empty (3 pages in use)
    before = s.state()
    with pytest.raises(NoPageError):
        s.begin_frame()
    assert s.state() == before
    s.rollback_last_frame()
    with pytest.raises(StateError):
        s.rollback_last_frame()         # double rollback
    # special pool: 2 pages x 4 slots = 8 tokens = 4 frames of 2
    s2 = StreamPages(0, 10, 2, 4, 20, 2)
    for _ in range(4):
        s2.begin_frame()
    before = s2.state()
    from oracle import SpecialFullError
    with pytest.raises(SpecialFullError):
        s2.begin_frame()
    assert s2.state() == before
    with pytest.raises(Exception):
        StreamPages(8, 64, 6, 16, 72, 10)   # pool smaller than S + W + 1


ops = st.lists(st.sampled_from(["frame", "defer_frame_commit",
                                "defer_frame_rollback", "reset"]),
               min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(S=st.integers(0, 3), W=st.integers(0, 4), Ns=st.integers(1, 3),
       Ps=st.integers(1, 5), extra=st.integers(0, 3), seq=ops)
def test_random_sequences_invariants(S, W, Ns, Ps, extra, seq):
    s = StreamPages(S, W, Ns, Ps, S + W + 1 + extra, 1000)
    evicted_total = 0
    specials_seen = 0
    for op in seq:
        if op == "reset":
            s.reset()
            evicted_total = 0
            specials_seen = 0
            continue
        if op == "frame":
            s.begin_frame()
            evicted_total += s.evict()
        else:
            before = s.state()
            s.set_defer(True)
            s.begin_frame()
            assert s.evict() == 0                  # deferred: nothing moves
            vis_deferred = s.visible_patch_pages()
            if op == "defer_frame_commit":
                evicted_total += s.execute_deferred_eviction()
                # the visible window does not depend on the deferral
                assert s.visible_patch_pages() == vis_deferred
            else:
                s.rollback_last_frame()
                assert s.state() == before         # exact inverse
            s.set_defer(False)
        used = s.scale + s.window
        assert len(s.free) + len(used) == s.pmax
        assert len(set(s.free) | set(used)) == s.pmax
        assert len(s.window) <= s.W
        assert len(s.scale) == min(S, s.frame_count)
        assert s.frame_count == len(s.scale) + len(s.window) + evicted_total
        assert s.n_special == Ns * s.frame_count   # specials never evicted
        assert s.n_special >= specials_seen or op in ("reset",
                                                      "defer_frame_rollback")
        specials_seen = s.n_special
        sp, last = s.visible_special_pages()
        if s.n_special:
            assert (len(sp) - 1) * Ps + last == s.n_special   # exact fill
            assert 1 <= last <= Ps


def test_oracle_cache_streams_have_disjoint_pages():
    c = OracleCache(layers=1, streams=3, heads=1, head_dim=1,
                    tokens_per_frame=5, num_special=2, special_page=3,
                    scale_frames=1, sliding_window=2, pmax=4, smax=10)
    rng = random.Random(0)
    for t in range(15):
        for b in range(3):
            drop = rng.random() < 0.3 and t > 0
            c.set_defer(b, drop)
            c.begin_frame(b)
            c.evict(b)
            if drop:
                c.rollback_last_frame(b)
            c.set_defer(b, False)
        tb = c.build_table()
        for b in range(3):
            p = tb.patch_ids[tb.patch_indptr[b]:tb.patch_indptr[b + 1]]
            q = tb.special_ids[tb.special_indptr[b]:tb.special_indptr[b + 1]]
            assert all(b * 4 <= x < (b + 1) * 4 for x in p)
            assert all(b * 10 <= x < (b + 1) * 10 for x in q)


def test_append_writes_expected_slots():
    """Specials first: rows [0, Ns) land in consecutive special slots across
    page boundaries; rows [Ns, T) fill the frame's patch page."""
    c = OracleCache(layers=1, streams=1, heads=1, head_dim=2,
                    tokens_per_frame=5, num_special=3, special_page=4,
                    scale_frames=1, sliding_window=1, pmax=3, smax=4,
                    storage=np.float32)
    for t in range(3):
        page, pos = c.begin_frame(0)
        k = np.arange(10, dtype=np.float32).reshape(5, 1, 2) + 100 * t
        c.append_frame(0, 0, k, -k)
        c.evict(0)
        for r, p in enumerate(pos):
            assert np.array_equal(c.special_pool[0][p // 4, 0, p % 4], k[r])
            assert np.array_equal(c.special_pool[0][p // 4, 1, p % 4], -k[r])
        assert np.array_equal(c.patch_pool[0][page, 0], k[3:])
