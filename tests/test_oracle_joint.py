"""Pins for joint prefill of several frames (oracle, CPU only).

Joint prefill: the first n frames are begun as one chunk and all n*T queries
attend together over a visible set that holds every frame of the chunk, so
earlier frames also see later ones (the scale frames' bidirectional context).
The paged oracle is checked against

* the float64 brute force over the dense history, where a chunk is current
  as a whole (random configurations, switches included);
* a closed relation: the queries of the chunk's last frame see exactly what
  single-frame streaming shows that frame, so their outputs agree, while the
  first frame's queries see more than in single-frame streaming;
* the bookkeeping of n single begins, and the exact undo of a chunk;

and a planted mistake in a copy of the page manager must be caught.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads as wl
from oracle import BruteForceHistory, OracleCache, StreamPages
from oracle.attention import paged_attention


def _qkv(w, b, frames):
    qs, ks, vs = zip(*(wl.frame_qkv(w, b, t, 0) for t in frames))
    return np.concatenate(qs), list(ks), list(vs)


def _joint_vs_brute(w, n, pages_cls=None, acc=np.float64):
    """Chunk of n frames, then single frames up to w.frames; worst difference
    to the brute force over all steps."""
    cache = OracleCache.for_workload(w)
    if pages_cls is not None:
        cache.streams = [pages_cls(w.scale_frames, w.sliding_window, w.num_special,
                                   w.special_page, w.pmax, w.smax,
                                   w.include_scale_frames, w.cross_frame_special)
                         for _ in range(w.streams)]
    hist = [BruteForceHistory(w.num_special, w.scale_frames, w.sliding_window,
                              w.include_scale_frames, w.cross_frame_special)
            for _ in range(w.streams)]
    steps = [list(range(n))] + [[t] for t in range(n, w.frames)]
    worst = 0.0
    for frames in steps:
        for b in range(w.streams):
            if len(frames) > 1:
                cache.begin_frames(b, len(frames))
            else:
                cache.begin_frame(b)
            cache.evict(b)
        table = cache.build_table()
        qs = []
        for b in range(w.streams):
            q, ks, vs = _qkv(w, b, frames)
            cache.append_frame(0, b, np.concatenate(ks), np.concatenate(vs))
            hist[b].push_chunk(ks, vs)
            qs.append(q)
        o, lse = paged_attention(cache.patch_pool[0], cache.special_pool[0], table,
                                 np.concatenate(qs), acc=acc)
        for b in range(w.streams):
            r0, r1 = int(table.qo_indptr[b]), int(table.qo_indptr[b + 1])
            assert r1 - r0 == len(frames) * w.tokens_per_frame
            o_ref, lse_ref = hist[b].attend(qs[b])
            worst = max(worst, float(np.abs(o[r0:r1] - o_ref).max()),
                        float(np.abs(lse[r0:r1] - lse_ref).max()))
    return worst


def test_scale_frames_jointly_match_brute_force():
    w = wl.TINY.replace(frames=10, streams=2, dtype="bf16")
    assert _joint_vs_brute(w, w.scale_frames) <= 1e-9


@settings(max_examples=50, deadline=None)
@given(S=st.integers(0, 3), W=st.integers(0, 4), Ns=st.integers(1, 3),
       P=st.integers(1, 7), Ps=st.integers(1, 5), B=st.integers(1, 2),
       n=st.integers(2, 5), after=st.integers(0, 6), seed=st.integers(0, 999),
       isf=st.booleans(), cfs=st.booleans())
def test_random_chunks_match_brute_force(S, W, Ns, P, Ps, B, n, after, seed,
                                         isf, cfs):
    S_eff = S if isf else 0
    if W == 0 and not cfs and S_eff == 0:
        return   # nothing would be visible
    if n - min(n, S_eff) > W:
        return   # refused: the window cannot hold the chunk
    w = wl.Workload("chunk", layers=1, heads=2, head_dim=8, dtype="fp32",
                    tokens_per_frame=P + Ns, num_special=Ns, special_page=Ps,
                    scale_frames=S, sliding_window=W, frames=n + after, streams=B,
                    seed=seed, include_scale_frames=isf, cross_frame_special=cfs)
    assert _joint_vs_brute(w, n) <= 1e-9


def test_last_chunk_frame_equals_single_streaming():
    """With n <= S the chunk's last frame sees frames 0..n-1, as does frame
    n-1 when frames are streamed one by one; frame 0 of the chunk sees all n
    frames, while streamed it sees only itself."""
    w = wl.TINY.replace(frames=4, heads=3)
    n = w.scale_frames
    joint = OracleCache.for_workload(w)
    joint.begin_frames(0, n)
    joint.evict(0)
    q, ks, vs = _qkv(w, 0, range(n))
    joint.append_frame(0, 0, np.concatenate(ks), np.concatenate(vs))
    oj, lj = paged_attention(joint.patch_pool[0], joint.special_pool[0],
                             joint.build_table(), q, acc=np.float64)
    single = OracleCache.for_workload(w)
    outs = []
    for t in range(n):
        single.begin_frame(0)
        single.evict(0)
        single.append_frame(0, 0, ks[t], vs[t])
        outs.append(paged_attention(single.patch_pool[0], single.special_pool[0],
                                    single.build_table(),
                                    q[t * w.tokens_per_frame:(t + 1) * w.tokens_per_frame],
                                    acc=np.float64))
    T = w.tokens_per_frame
    assert np.abs(oj[(n - 1) * T:] - outs[-1][0]).max() < 1e-12
    assert np.abs(lj[(n - 1) * T:] - outs[-1][1]).max() < 1e-12
    assert np.abs(lj[:T] - outs[0][1]).min() > 1e-6   # frame 0 sees more keys


def test_chunk_bookkeeping_is_n_single_begins():
    a = StreamPages(3, 2, 2, 3, 8, 6)
    b = StreamPages(3, 2, 2, 3, 8, 6)
    a.begin_frames(4)
    for _ in range(4):
        b.begin_frame()
    assert a.state() == b.state()
    assert [p for p, _ in a.current_frames()] == a.scale + a.window
    assert a.current_frames()[3][1] == [6, 7]
    before = StreamPages(3, 2, 2, 3, 8, 6).state()
    a.rollback_last_frame()
    assert a.state() == before


def test_chunk_limits():
    s = StreamPages(1, 2, 1, 4, 4, 4)
    with pytest.raises(Exception):
        s.begin_frames(4)     # 3 window frames, W = 2
    s.begin_frames(3)
    s.evict()
    assert s.stats()["live_pages"] == 2
    s2 = StreamPages(2, 2, 1, 4, 5, 1)
    with pytest.raises(Exception):
        s2.begin_frames(5)    # 5 specials, one page of 4
    assert s2.state() == StreamPages(2, 2, 1, 4, 5, 1).state()


class _ChunkSpecialsOverlap(StreamPages):
    def begin_frames(self, n):
        frames = super().begin_frames(n)
        # every frame of the chunk writes its specials over the first's
        self.cur = [(p, frames[0][1]) for p, _ in frames]
        return self.cur


def test_planted_chunk_mistake_is_caught():
    w = wl.TINY.replace(frames=6, heads=2)
    assert _joint_vs_brute(w, w.scale_frames) <= 1e-9
    assert _joint_vs_brute(w, w.scale_frames, pages_cls=_ChunkSpecialsOverlap) > 1e-3
