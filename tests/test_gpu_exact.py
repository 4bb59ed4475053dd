"""Token-exact GPU checks at full size.

With N(0,1) data and ~20 000 visible tokens, one token dropped, added or read
from the wrong place moves the log-sum-exp by about 1/Lkv (5e-5), far inside
the 1e-3 bound of the ordinary parity tests.  These tests use inputs whose
attention has a closed form that exposes every token
(``workloads.frame_qkv_coded``): every key of a head is the same vector, so
each query's weights are exactly 1/Lkv, and every value row is one-hot by the
token's class.  The visible set comes from the oracle's table and pools; the
GPU result must give lse = s + ln(Lkv) within 1e-5 and the exact count of
visible tokens of every class (see ``_parity._exact_check``).  This pins the
page lookup of the kernel (patch pages, the special head and tail, the last
page fill of [p1] "How the Paged KV Cache Attention Mechanism Enables Long
Sequence Inference in LingBot-Map", §Building the Visible Page Table) and, on
the one-launch path, the rows of the current frame read from k/v.
"""
import pytest

import workloads as wl
from _parity import run

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-5


def _ok_exact(worst, checks):
    print(f"exact: lse {worst.exact_lse:.3g} count {worst.exact_count:.3g} "
          f"o/bound {worst.exact_o:.3g} over {worst.exact_checked} checks, "
          f"fused steps {worst.fused_steps}", flush=True)
    assert worst.exact_checked == checks
    assert worst.exact_lse <= LSE_TOL
    assert worst.exact_count < 0.5
    assert worst.exact_o <= 1.0


def test_exact_main_224_fused_every_frame(gpu):
    """Every frame of the 224x224 workload through psw_append_attention (one
    launch per frame), pools bit-exact where the window fills and at the end."""
    w = wl.MAIN
    worst = run(w, exact=True, fused=True, pools_at=[71, 319], log_every=64)
    _ok_exact(worst, w.frames)
    assert worst.fused_steps == w.frames


def test_exact_main_224_separate_every_frame(gpu):
    """The same through psw_append_frames + psw_attention."""
    w = wl.MAIN
    _ok_exact(run(w, exact=True, log_every=64), w.frames)


def test_exact_nocross_224_fused_every_frame(gpu):
    """Without cross-frame specials: the special head and tail ranges."""
    w = wl.NOCROSS
    worst = run(w, exact=True, fused=True, log_every=64)
    _ok_exact(worst, w.frames)
    assert worst.fused_steps == w.frames


def test_exact_keyframe_224_fused(gpu):
    """Deferred eviction and rollback: every frame of the first 300 (126
    keyframe transitions; from frame 243 on the window is full and a deferred
    frame holds W + 1 window pages) and the last frame."""
    w = wl.KEYFRAME
    kf = [wl.keyframe_mask(w, 0)]
    sample = set(range(300)) | {w.frames - 1}
    worst = run(w, keyframes=kf, exact=True, fused=True,
                attend=lambda t: t in sample, pools_at=[w.frames - 1], log_every=100)
    _ok_exact(worst, len(sample))


def test_exact_large_518x378_sampled(gpu):
    """Four ragged 1005-row streams (about 73 000 visible tokens each at the
    end), frames around the window filling and the last."""
    w = wl.LARGE
    sample = {0, 7, 8, 71, 72, 199}
    worst = run(w, exact=True, fused=True, attend=lambda t: t in sample, log_every=50)
    _ok_exact(worst, len(sample))


def test_exact_stack_224x24_sampled(gpu):
    """24 layers sharing one table: the first and the last layer."""
    w = wl.STACK.replace(frames=80)
    sample = {0, 71, 72, 79}
    worst = run(w, exact=True, fused=True, attend=lambda t: t in sample,
                layers_checked=[0, 23])
    _ok_exact(worst, 2 * len(sample))
    assert worst.fused_steps == w.frames * w.layers


def _one_split_beyond_table():
    # 134-token frames (128 patches), 500 frames, nothing evicted: 67 000 keys
    # (1047 tiles of 64) at the last frame, more than the 1024 tiles the
    # per-workgroup group table of the kernel holds, while the frame stays
    # under the one-launch limit of 2^28 query-key-head scores.  16 heads:
    # 1024 value classes, so each count (about 65) stays well below 2^8, as
    # the count check needs.
    return wl.NOEVICT.replace(name="noevict_1split", tokens_per_frame=134, frames=500,
                              sliding_window=500)


@pytest.mark.parametrize("fused", [True, False])
def test_exact_one_split_beyond_the_group_table(gpu, fused):
    """One KV split per stream (max_kv_splits = 1) over more key tiles than the
    group table holds: the tiles past it take the row-by-row page lookup (on
    the one-launch path with the current frame's rows, the last ones, read
    from k/v).  Every visible token must be counted once."""
    w = _one_split_beyond_table()
    last = range(w.frames - 4, w.frames)
    worst = run(w, exact=True, fused=fused, attend=lambda t: t in last,
                cache_kw={"max_kv_splits": 1}, on_plan=_one_split)
    _ok_exact(worst, len(last))
    if fused:
        assert worst.fused_steps == w.frames


def _one_split(t, gc):
    items, splits = gc.plan_info()
    assert splits == 1, (t, items, splits)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_exact_long_video(gpu, fused):
    """A 3 000-frame video of the 224x224 geometry: every patch page goes
    round the free stack about 40 times and the special pool grows to 18 000
    tokens (36 432 visible keys at the end).  Token-exact at frames 999,
    1 999 and 2 999; pools bit-exact at the end.  The special pages listed
    grow with the video (1 125 at the end); the plan gives them as two runs
    of consecutive page ids, so it keeps fitting the kernel arguments and, on
    psw_append_attention, every frame runs as one launch.  Both call forms
    and both workgroup shapes (4 waves early, 8 once the frame splits its
    keys widely) read the special pages from the two runs."""
    w = wl.MAIN.replace(name="long_224", frames=3_000)
    checked = (999, 1999, 2999)
    waves, late = {}, set()

    def on_plan(t, gc):
        waves.setdefault(gc.plan_waves(), t)
        if t >= 2_520:   # 945+ special pages listed: the list alone is too long
            late.add(gc.plan_waves())

    worst = run(w, exact=True, fused=fused, attend=lambda t: t in checked,
                pools_at=[w.frames - 1], log_every=500, on_plan=on_plan)
    print("first frame of each workgroup shape:", waves, "from frame 2520:", late,
          flush=True)
    _ok_exact(worst, len(checked))
    if fused:
        assert worst.fused_steps == w.frames


# Small special pages with cross-frame specials off: the table lists every
# visible frame's special pages, a head run (the scale frames') and a tail run
# (the window frames'), and the list soon pushes the plan past the 944 ints of
# the one-launch kernel's arguments, while the rest of the plan (patch pages,
# work items, append segments) still fits; the plan then gives each stream's
# special pages as its two runs of consecutive ids.
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("B,T,num_special,page,window,frames,shape", [
    # two streams of 2 376 keys at the end, up to 10 splits: 4 waves
    (2, 22, 6, 1, 100, 150, 4),
    # one stream of 20 960 keys, 16 splits: 8 waves; pages of 2 tokens hold
    # the 25 specials of alternate frames from a page's first or second slot
    (1, 262, 25, 2, 72, 120, 8),
], ids=["two_streams_4waves", "one_stream_8waves"])
def test_exact_special_page_runs(gpu, fused, B, T, num_special, page, window, frames,
                                 shape):
    """Token-exact at every frame, on both call forms, in the workgroup shape
    named at the last frame; the one-launch path runs every frame as one
    launch, and the dense check path gathers the same tokens at the last frame.
    A frame counts as long when its special and patch page lists and 16 ints
    per work item alone exceed 944 ints: the plan of such a frame can only fit
    with the runs."""
    w = wl.Workload(f"special_runs_{B}x{T}", layers=1, heads=16, head_dim=64,
                    dtype="bf16", tokens_per_frame=T, num_special=num_special,
                    special_page=page, scale_frames=8, sliding_window=window,
                    frames=frames, streams=B, cross_frame_special=False, seed=T)
    long_list = {}

    def on_plan(t, gc):
        pt = gc.page_table()
        items, _ = gc.plan_info()
        if len(pt["special_ids"]) + len(pt["patch_ids"]) + 16 * items > 944:
            long_list[t] = (gc.plan_waves(), gc.plan_fused())

    worst = run(w, exact=True, fused=fused, on_plan=on_plan,
                dense_at=[] if fused else [frames - 1], pools_at=[frames - 1])
    late = sorted(long_list)
    print(f"{len(late)} long frames from frame {late[:1]}: shapes "
          f"{sorted({s for s, _ in long_list.values()})}, "
          f"fused {sum(f for _, f in long_list.values())}", flush=True)
    _ok_exact(worst, frames)
    assert len(late) >= 20 and late[-1] == frames - 1
    assert all(f for _, f in long_list.values()), [t for t in late if not long_list[t][1]]
    assert long_list[frames - 1][0] == shape
    if fused:
        assert worst.fused_steps == frames
    else:
        from test_gpu_dense import _ok_dense
        _ok_dense(worst)
