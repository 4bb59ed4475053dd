"""Pins for the oracle's paged attention (CPU only).

The paged oracle (page manager + gather + float32 softmax) is checked against
* the float64 brute force over the dense history with a frame-rule mask,
* library attention (torch's scaled_dot_product_attention on the CPU, float64)
  in the special cases that reduce to it (first frame; no eviction),
* closed forms (identical keys -> uniform weights and lse = s + ln Lkv;
  constant values -> o = v), and
* invariances (page order in the table, independence of heads),
and planted mistakes in a copy of the page manager must be caught.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import workloads as wl
from oracle import BruteForceHistory, OracleCache, StreamPages
from oracle.attention import paged_attention
from oracle.stream import stream_frames


def _run_vs_brute(w, keyframes=None, acc=np.float32, tol=1e-5,
                  pages_cls=None, n_frames=None):
    cache = OracleCache.for_workload(w)
    if pages_cls is not None:
        cache.streams = [pages_cls(w.scale_frames, w.sliding_window,
                                   w.num_special, w.special_page, w.pmax,
                                   w.smax, w.include_scale_frames,
                                   w.cross_frame_special)
                         for _ in range(w.streams)]
    hist = [BruteForceHistory(w.num_special, w.scale_frames, w.sliding_window,
                              w.include_scale_frames, w.cross_frame_special)
            for _ in range(w.streams)]
    inputs = lambda b, t, l: wl.frame_qkv(w, b, t, l)
    n = n_frames or w.frames
    worst = 0.0
    for step in stream_frames(cache, n, inputs, keyframes=keyframes, acc=acc):
        t = step["t"]
        for b in range(w.streams):
            q, k, v = inputs(b, t, 0)
            hist[b].push(k, v)
            o_ref, lse_ref = hist[b].attend(q)
            o, lse = step["out"][0]
            r0 = int(step["table"].qo_indptr[b])
            worst = max(worst,
                        np.abs(o[r0:r0 + w.tokens_per_frame] - o_ref).max(),
                        np.abs(lse[r0:r0 + w.tokens_per_frame] - lse_ref).max())
            if keyframes is not None and not keyframes[b][t]:
                hist[b].drop_current()
    return worst


def test_tiny_matches_brute_force():
    assert _run_vs_brute(wl.TINY) <= 1e-5


def test_tiny_bf16_keyframes_matches_brute_force():
    w = wl.TINY.replace(dtype="bf16", frames=30, keyframe_p=0.4, seed=3)
    kf = [wl.keyframe_mask(w, 0)]
    assert not kf[0].all() and kf[0].any()
    assert _run_vs_brute(w, keyframes=kf) <= 1e-5


@settings(max_examples=60, deadline=None)
@given(S=st.integers(0, 3), W=st.integers(0, 4), Ns=st.integers(1, 4),
       P=st.integers(1, 9), Ps=st.integers(1, 6), B=st.integers(1, 3),
       frames=st.integers(1, 14), kfp=st.sampled_from([None, 0.5]),
       seed=st.integers(0, 1000), isf=st.booleans(), cfs=st.booleans())
def test_random_configs_match_brute_force(S, W, Ns, P, Ps, B, frames, kfp,
                                          seed, isf, cfs):
    """Includes both switches: no scale frames, no cross-frame specials."""
    if W == 0 and not cfs and (S == 0 or not isf):
        return   # nothing would be visible: refused by the page manager
    w = wl.Workload("rand", layers=1, heads=2, head_dim=8, dtype="fp32",
                    tokens_per_frame=P + Ns, num_special=Ns, special_page=Ps,
                    scale_frames=S, sliding_window=W, frames=frames, streams=B,
                    keyframe_p=kfp, seed=seed, include_scale_frames=isf,
                    cross_frame_special=cfs)
    kf = None if kfp is None else [wl.keyframe_mask(w, b) for b in range(B)]
    assert _run_vs_brute(w, keyframes=kf, acc=np.float64, tol=1e-9) <= 1e-9


def _sdpa64(q, k, v):
    """torch's library attention, CPU, float64.  q [T, H, D], k/v [N, H, D]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(
        x.transpose(1, 0, 2))).double()
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    return o.numpy().transpose(1, 0, 2)


def test_first_frame_is_plain_attention():
    """At the first frame the visible set is the frame itself."""
    w = wl.MAIN.replace(heads=4)
    cache = OracleCache.for_workload(w)
    q, k, v = wl.frame_qkv(w, 0, 0, 0)
    cache.begin_frame(0)
    cache.evict(0)
    cache.append_frame(0, 0, k, v)
    o, _ = paged_attention(cache.patch_pool[0], cache.special_pool[0],
                           cache.build_table(), q, acc=np.float64)
    f = wl.bf16_bits_to_f32
    ref = _sdpa64(f(q), f(k), f(v))
    assert np.abs(o - ref).max() < 1e-12


def test_no_eviction_is_dense_history_attention():
    """With a window longer than the video nothing is evicted: attention over
    the whole concatenated history (the pages' SDPA contrast)."""
    w = wl.TINY.replace(sliding_window=20, frames=9, heads=3)
    cache = OracleCache.for_workload(w)
    ks, vs = [], []
    for t in range(w.frames):
        q, k, v = wl.frame_qkv(w, 0, t, 0)
        cache.begin_frame(0)
        cache.evict(0)
        cache.append_frame(0, 0, k, v)
        ks.append(k)
        vs.append(v)
        o, _ = paged_attention(cache.patch_pool[0], cache.special_pool[0],
                               cache.build_table(), q, acc=np.float64)
        ref = _sdpa64(q, np.concatenate(ks), np.concatenate(vs))
        assert np.abs(o - ref).max() < 1e-12


def test_identical_keys_closed_form():
    """All keys equal: uniform weights, o = mean of the visible values,
    lse = q.k/sqrt(D) + ln(Lkv)."""
    w = wl.TINY.replace(frames=8)
    cache = OracleCache.for_workload(w)
    rng = np.random.default_rng(1)
    key = rng.standard_normal((w.heads, w.head_dim)).astype(np.float32)
    for t in range(w.frames):
        q, _, v = wl.frame_qkv(w, 0, t, 0)
        k = np.broadcast_to(key, v.shape).copy()
        cache.begin_frame(0)
        cache.evict(0)
        cache.append_frame(0, 0, k, v)
    tb = cache.build_table()
    o, lse = paged_attention(cache.patch_pool[0], cache.special_pool[0], tb, q,
                             acc=np.float64)
    lkv = tb.kv_len(0, w.patch_page, w.special_page)
    # visible values, collected by hand from the frame rules: frames 0,1
    # (scale) and 4..7 (window) patches, specials of all frames
    vis = []
    for t in range(w.frames):
        _, _, v = wl.frame_qkv(w, 0, t, 0)
        vis.append(v[:w.num_special])
        if t < 2 or t >= 4:
            vis.append(v[w.num_special:])
    vis = np.concatenate(vis).astype(np.float64)
    assert vis.shape[0] == lkv == 6 * 16 + 8 * 6
    s = np.einsum("thd,hd->th", q.astype(np.float64), key) / np.sqrt(w.head_dim)
    assert np.abs(lse - (s + np.log(lkv))).max() < 1e-9
    assert np.abs(o - vis.mean(axis=0)[None]).max() < 1e-9


def test_constant_values_and_order_and_heads():
    w = wl.TINY.replace(frames=10, heads=3)
    cache = OracleCache.for_workload(w)
    for t in range(w.frames):
        q, k, v = wl.frame_qkv(w, 0, t, 0)
        cache.begin_frame(0)
        cache.evict(0)
        cache.append_frame(0, 0, k, np.full_like(v, 0.75))
    tb = cache.build_table()
    o, lse = paged_attention(cache.patch_pool[0], cache.special_pool[0], tb, q,
                             acc=np.float64)
    assert np.abs(o - 0.75).max() < 1e-12
    # permuting the listed pages leaves the result unchanged
    perm = type(tb)(**vars(tb))
    perm.patch_ids = tb.patch_ids[::-1].copy()
    o2, lse2 = paged_attention(cache.patch_pool[0], cache.special_pool[0], perm,
                               q, acc=np.float64)
    assert np.abs(lse2 - lse).max() < 1e-12
    # heads are independent: changing head 2's queries leaves heads 0, 1
    q3 = q.copy()
    q3[:, 2] *= -3
    _, lse3 = paged_attention(cache.patch_pool[0], cache.special_pool[0], tb,
                              q3, acc=np.float64)
    assert np.array_equal(lse3[:, :2], lse[:, :2])
    assert not np.allclose(lse3[:, 2], lse[:, 2])


# -- planted mistakes: a wrong page manager must fail the brute-force pin ----

class _WindowOffByOne(StreamPages):
    def visible_patch_pages(self):
        start = max(0, len(self.window) - self.W + 1)
        return list(self.scale) + list(self.window[start:])


class _ScaleIsRecent(StreamPages):
    def begin_frame(self):
        page, pos = super().begin_frame()
        return page, pos

    def visible_patch_pages(self):
        win = self.window[max(0, len(self.window) - self.W):]
        return list(win[-self.S:]) + list(win)


class _DropsOldSpecials(StreamPages):
    def visible_special_segments(self):
        # forgets the first special page's tokens once a second page exists
        return [(max(a, self.Ps), b) if self.n_special > self.Ps else (a, b)
                for a, b in super().visible_special_segments()]


class _LastPageFull(StreamPages):
    def visible_special_segments(self):
        # reads the last special page whole, stale slots included
        segs = super().visible_special_segments()
        if segs:
            a, b = segs[-1]
            segs[-1] = (a, -(-b // self.Ps) * self.Ps)
        return segs


class _KeepsEvictedSpecials(StreamPages):
    def visible_special_segments(self):
        # ignores the switch: every kept frame's specials stay visible
        return [(0, self.n_special)] if self.n_special else []


@pytest.mark.parametrize("cls", [_WindowOffByOne, _ScaleIsRecent,
                                 _DropsOldSpecials, _LastPageFull])
def test_planted_mistakes_are_caught(cls):
    w = wl.TINY.replace(frames=12)
    assert _run_vs_brute(w, pages_cls=cls) > 1e-3


def test_planted_switch_mistake_is_caught():
    w = wl.TINY.replace(frames=12, cross_frame_special=False)
    assert _run_vs_brute(w) <= 1e-5
    assert _run_vs_brute(w, pages_cls=_KeepsEvictedSpecials) > 1e-3


def test_switches_off_before_any_eviction_change_nothing():
    """While nothing has been evicted the switches change nothing: without
    cross-frame specials for the first S + W frames; without scale frames
    (every frame a window frame) for the first W frames."""
    for kw, horizon in (({"cross_frame_special": False},
                         wl.TINY.scale_frames + wl.TINY.sliding_window),
                        ({"include_scale_frames": False}, wl.TINY.sliding_window)):
        base = wl.TINY.replace(frames=horizon + 1)
        w = base.replace(**kw)
        c0, c1 = OracleCache.for_workload(base), OracleCache.for_workload(w)
        for t in range(horizon):
            for c in (c0, c1):
                c.begin_frame(0)
                c.evict(0)
            t0, t1 = c0.build_table(), c1.build_table()
            assert t0.kv_len(0, base.patch_page, base.special_page) == \
                t1.kv_len(0, w.patch_page, w.special_page)
        # one frame more and the visible sets differ
        for c in (c0, c1):
            c.begin_frame(0)
            c.evict(0)
        assert c0.build_table().kv_len(0, base.patch_page, base.special_page) != \
            c1.build_table().kv_len(0, w.patch_page, w.special_page)
