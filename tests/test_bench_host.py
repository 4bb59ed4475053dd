"""Host-side arithmetic of bench.py (no GPU): which frames carry timing
events, the algorithmic bytes and flops the roofline divides, and the roof
that binds.  The visible token counts come from the library's own host
bookkeeping and are checked against their closed form."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_timed_frames_cover_every_frame_once_in_a_full_rotation():
    w = wl.MAIN
    seen = []
    for step in range(bench.PROFILE_EVERY):
        fr = list(bench.timed_frames(w, step))
        # one frame per block of PROFILE_EVERY frames, evenly spaced
        assert all(b - a == bench.PROFILE_EVERY for a, b in zip(fr, fr[1:]))
        seen += fr
    assert sorted(seen) == list(range(w.frames))


def test_schedule_matches_closed_form():
    # scale + window pages of P patch tokens, and every frame's Ns specials
    # (cross-frame specials on): Lkv(t) = min(t + 1, S + W) * P + (t + 1) * Ns
    w = wl.MAIN
    kv, kf = bench.step_schedule(w)
    assert kf is None
    P = w.tokens_per_frame - w.num_special
    for t, row in enumerate(kv):
        want = min(t + 1, w.scale_frames + w.sliding_window) * P + (t + 1) * w.num_special
        assert row == [want], t
    assert kv[-1] == [20352]


def test_algorithmic_work_per_frame():
    w = wl.MAIN
    kv, _ = bench.step_schedule(w)
    e, T, H, D = w.elem_bytes, w.tokens_per_frame, w.heads, w.head_dim
    b, a, f = bench.algorithmic_work(w, kv, [319])
    lkv = kv[319][0]
    assert b == lkv * H * D * 2 * e + 2 * T * H * D * e + T * H * 4
    assert a == 2 * T * H * D * 2 * e
    assert f == 4 * T * lkv * D * H
    # the whole step is the sum of its frames
    tot = bench.algorithmic_work(w, kv)
    parts = [bench.algorithmic_work(w, kv, [t]) for t in range(w.frames)]
    assert tot == tuple(sum(p[i] for p in parts) for i in range(3))
    # the step totals quoted for the 224x224 workload: 5.958 TFLOP
    assert round(tot[2] / 1e12, 3) == 5.958


def test_roofline_bound_follows_the_ridge():
    ridge = bench.MFMA_BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert ridge == pytest.approx(312.5)
    assert bench.roofline_bound(300.0, 1.0, "bf16") == "hbm"
    assert bench.roofline_bound(320.0, 1.0, "bf16") == "mfma"
    for name, bound in (("main_224", "hbm"), ("large_518x378", "mfma")):
        w = wl.ALL[name]
        kv, _ = bench.step_schedule(w)
        b, _, f = bench.algorithmic_work(w, kv)
        assert bench.roofline_bound(f, b, w.dtype) == bound, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
