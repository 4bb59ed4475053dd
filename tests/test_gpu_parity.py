"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bit-exact: page tables, free lists, stats and the bytes the append kernel
writes into the pools.  Attention: max-abs <= 1e-2 on o and <= 1e-3 on lse
for bf16 (float accumulation), <= 1e-4 for float32, and a relative Frobenius
error <= 2e-2 on o.
"""
import numpy as np
import pytest

import workloads as wl
from _parity import (BF16_TOL_LSE, BF16_TOL_O, BF16_TOL_REL, FP32_TOL, run)

pytestmark = pytest.mark.gpu


def _ok_bf16(worst):
    print(f"worst o {worst.o:.3g} lse {worst.lse:.3g} rel {worst.rel:.3g} "
          f"over {worst.checked} checks", flush=True)
    assert worst.checked > 0
    assert worst.o <= BF16_TOL_O
    assert worst.lse <= BF16_TOL_LSE
    assert worst.rel <= BF16_TOL_REL


def test_tiny_fp32_every_frame(gpu):
    w = wl.TINY
    worst = run(w, pools_at=range(w.frames))
    print(worst, flush=True)
    assert worst.checked == w.frames
    assert worst.o <= FP32_TOL and worst.lse <= FP32_TOL


def test_fp32_three_streams_keyframes_every_frame(gpu):
    """The float32 kernel over three streams whose keyframe masks differ, so
    the streams' histories and visible lengths grow apart (and a rolled-back
    frame leaves its stream out of the next tables)."""
    w = wl.TINY.replace(streams=3, frames=16, keyframe_p=0.5, heads=3)
    kf = [wl.keyframe_mask(w, b) for b in range(w.streams)]
    worst = run(w, keyframes=kf, pools_at=[w.frames - 1])
    print(worst, flush=True)
    assert worst.checked == w.frames
    assert worst.o <= FP32_TOL and worst.lse <= FP32_TOL


SMALL_BF16 = [
    # T, Ns, Ps, S, W, H, frames, B: several 64-key tiles and ragged tails
    dict(tokens_per_frame=22, num_special=6, special_page=8, scale_frames=2,
         sliding_window=4, heads=2, frames=40, streams=1),
    dict(tokens_per_frame=106, num_special=6, special_page=16, scale_frames=3,
         sliding_window=5, heads=4, frames=30, streams=1),
    dict(tokens_per_frame=70, num_special=5, special_page=3, scale_frames=1,
         sliding_window=3, heads=3, frames=25, streams=3),
    dict(tokens_per_frame=17, num_special=1, special_page=1, scale_frames=0,
         sliding_window=6, heads=1, frames=30, streams=2),
    dict(tokens_per_frame=40, num_special=6, special_page=16, scale_frames=2,
         sliding_window=0, heads=2, frames=20, streams=1),
    dict(tokens_per_frame=333, num_special=6, special_page=16, scale_frames=2,
         sliding_window=3, heads=2, frames=12, streams=2),
]


@pytest.mark.parametrize("i", range(len(SMALL_BF16)))
def test_small_bf16_every_frame(gpu, i):
    w = wl.Workload(f"small{i}", layers=2, head_dim=64, dtype="bf16", seed=i,
                    **SMALL_BF16[i])
    worst = run(w, pools_at=[w.frames - 1])
    _ok_bf16(worst)


def test_per_stream_append_then_attention(gpu):
    """Frames written stream by stream (psw_append_frame): the plan then
    reaches the device with the attention call itself."""
    w = wl.Workload("per_stream", layers=2, head_dim=64, dtype="bf16", seed=21,
                    **SMALL_BF16[2])
    _ok_bf16(run(w, pools_at=[w.frames - 1], per_stream_append=True))


SWITCHES = [
    # (geometry index, switches): head and tail ranges starting mid-page,
    # page size 3 and 1, three streams, keyframes
    (0, {"cross_frame_special": False}),
    (2, {"cross_frame_special": False}),
    (3, {"cross_frame_special": False}),
    (1, {"include_scale_frames": False}),
    (5, {"include_scale_frames": False, "cross_frame_special": False}),
]


@pytest.mark.parametrize("i", range(len(SWITCHES)))
def test_switches_small_every_frame(gpu, i):
    """Without cross-frame specials (only visible frames' specials attend)
    and without scale frames."""
    g, sw = SWITCHES[i]
    w = wl.Workload(f"switch{i}", layers=2, head_dim=64, dtype="bf16", seed=40 + i,
                    **SMALL_BF16[g], **sw)
    _ok_bf16(run(w, pools_at=[w.frames - 1]))


def test_switches_keyframes_ragged(gpu):
    w = wl.Workload("switch_kf", layers=1, heads=2, head_dim=64, dtype="bf16",
                    tokens_per_frame=70, num_special=6, special_page=16,
                    scale_frames=2, sliding_window=5, frames=40, streams=3,
                    keyframe_p=0.5, seed=12, cross_frame_special=False)
    kf = [wl.keyframe_mask(w, b) for b in range(w.streams)]
    _ok_bf16(run(w, keyframes=kf, pools_at=[w.frames - 1]))


def test_main_224_no_cross_frame_specials_sampled(gpu):
    """Full size without cross-frame specials: from frame 72 on the evicted
    frames' specials drop out of the visible set."""
    w = wl.MAIN.replace(cross_frame_special=False)
    sample = {0, 71, 72, 73, 150, 319}
    _ok_bf16(run(w, attend=lambda t: t in sample, heads_checked=[0, 15]))


def test_small_bf16_keyframes_ragged(gpu):
    """Different keyframe masks per stream: the streams' visible lengths
    differ (a ragged batch) and rolled-back frames must leave no trace."""
    w = wl.Workload("ragged", layers=1, heads=2, head_dim=64, dtype="bf16",
                    tokens_per_frame=70, num_special=6, special_page=16,
                    scale_frames=2, sliding_window=5, frames=40, streams=3,
                    keyframe_p=0.5, seed=11)
    kf = [wl.keyframe_mask(w, b) for b in range(w.streams)]
    worst = run(w, keyframes=kf, pools_at=[w.frames - 1])
    _ok_bf16(worst)


def test_peaked_softmax(gpu):
    """q scaled by 8: the softmax is peaked and |o| reaches a few units.

    bf16 arithmetic then bounds the error per element by one rounding of
    the output (2^-9 |o|) plus the rounding of the weights before the PV
    product (each weight within 2^-9 relative, so at most 2^-9 max|v|):
    |o - o_ref| <= 2^-9 (|o_ref| + max|v|), doubled for margin.  The lse
    does not see either rounding and keeps its 1e-3 bound.  The plan splits
    the keys of the late frames 33 to 64 ways."""
    w = wl.MAIN.replace(frames=80, heads=4)
    splits = {}

    def record(t, gc):
        splits[t] = gc.plan_info()[1]
    worst = run(w, q_scale=8.0, attend=lambda t: t in (0, 5, 40, 71, 72, 79),
                on_plan=record)
    print(worst, "splits at frame 79:", splits[79], flush=True)
    assert worst.checked == 6
    # 4 heads over ~19k keys: 33 to 64 KV splits, the merge's widest shape
    assert 33 <= splits[79] <= 64
    assert worst.scaled <= 2.0 ** -8
    assert worst.lse <= BF16_TOL_LSE
    assert worst.rel <= BF16_TOL_REL


def test_permuted_table_same_result(gpu):
    """Reversing the order of the listed pages must not change the result."""
    w = wl.TINY.replace(dtype="bf16", frames=14, heads=2, streams=2)

    def reverse(t, tbl):
        tbl = {k: v.copy() for k, v in tbl.items()}
        for b in range(2):
            s, e = tbl["patch_indptr"][b], tbl["patch_indptr"][b + 1]
            tbl["patch_ids"][s:e] = tbl["patch_ids"][s:e][::-1]
        return tbl
    _ok_bf16(run(w, table_hook=reverse))


def test_main_224_sampled(gpu):
    """The 262 tok/frame workload, all 320 frames streamed; attention
    checked on a spread of frames (window filling, full, steady state)."""
    w = wl.MAIN
    sample = {0, 1, 2, 7, 8, 9, 31, 63, 64, 70, 71, 72, 73, 100, 150, 200,
              255, 256, 300, 318, 319}
    worst = run(w, attend=lambda t: t in sample, pools_at=[71, 319],
                log_every=64)
    _ok_bf16(worst)


def test_stack_224x24_sampled(gpu):
    w = wl.STACK
    sample = {0, 70, 71, 72, 319}
    worst = run(w, attend=lambda t: t in sample, layers_checked=[0, 23],
                pools_at=[319], log_every=64)
    _ok_bf16(worst)


def test_keyframe_224_sampled(gpu):
    w = wl.KEYFRAME
    kf = [wl.keyframe_mask(w, 0)]
    trans = [t for t in range(1, 300) if kf[0][t] != kf[0][t - 1]][:12]
    sample = set(trans) | {0, w.frames - 1}
    worst = run(w, keyframes=kf, attend=lambda t: t in sample,
                pools_at=[w.frames - 1], log_every=200)
    _ok_bf16(worst)


def test_interval_224_sampled(gpu):
    """Keyframe interval 4 (frames 0, 4, 8, ... kept, the others attended
    with eviction deferred and rolled back): tables, free lists and stats on
    every frame, attention on transitions around the window filling up and
    the last frames."""
    w = wl.INTERVAL
    kf = [wl.keyframe_mask(w)]
    sample = {0, 1, 3, 4, 5, 55, 100, 196, 197, 199}
    worst = run(w, keyframes=kf, attend=lambda t: t in sample, heads_checked=[0, 9],
                pools_at=[199])
    _ok_bf16(worst)


def test_large_518x378_sampled(gpu):
    w = wl.LARGE
    sample = {0, 7, 8, 71, 72, 199}
    worst = run(w, attend=lambda t: t in sample, heads_checked=[0, 15],
                pools_at=[199], log_every=50)
    _ok_bf16(worst)


def test_constant_values_closed_form(gpu):
    """Constant V gives o = V exactly (up to the bf16 output rounding)."""
    import torch
    from paged_sliding_window_append_amd import Cache
    w = wl.MAIN.replace(frames=75, heads=2)
    c = Cache.for_workload(w)
    for t in range(w.frames):
        c.begin_frame(0)
        c.evict_frames(0)
        c.build_visible_page_table()
        c.plan()
        q, k, _ = wl.frame_qkv_tensors(w, 0, t, 0)
        v = torch.full_like(k, 0.375)
        c.append_frames(0, k.cuda(), v.cuda())
        o, lse = c.attention(0, q.cuda())
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0.375)
    assert torch.isfinite(lse).all()


def test_empty_table_is_a_no_op(gpu):
    import torch
    from paged_sliding_window_append_amd import Cache
    c = Cache.for_workload(wl.TINY.replace(dtype="bf16"))
    c.build_visible_page_table()
    c.plan()
    assert c.plan_info() == (0, 0)
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    c.attention(0, q)
    torch.cuda.synchronize()


def test_noevict_224_sampled(gpu):
    """No eviction (window as long as the 320-frame video): the whole
    history stays visible, 83 840 tokens at the last frame; every row and
    head of the last frame also against the dense float32 path."""
    w = wl.NOEVICT
    sample = {0, 71, 72, 200, 319}
    worst = run(w, attend=lambda t: t in sample, heads_checked=[0, 13],
                pools_at=[319], dense_at={319})
    _ok_bf16(worst)
    assert worst.dense_checked == 1
    assert worst.cross_o <= BF16_TOL_O and worst.cross_lse <= BF16_TOL_LSE


def test_reset_between_videos(gpu):
    """A cache reset between videos ([p2] §Manual Cache Control): stream 1 is
    emptied after 14 frames and starts a new video on pages that still hold
    the old one's K/V, while stream 0 carries on.  Every frame must match an
    oracle whose stream 1 was reset at the same point, and the tables must
    equal its tables."""
    import torch
    from oracle.attention import paged_attention
    from oracle.cache import OracleCache
    from paged_sliding_window_append_amd import Cache
    w = wl.Workload("reset", layers=1, heads=2, head_dim=64, dtype="bf16",
                    tokens_per_frame=70, num_special=6, special_page=8, scale_frames=2,
                    sliding_window=4, frames=30, streams=2, seed=33)
    gc = Cache.for_workload(w, device="cuda:0")
    oc = OracleCache.for_workload(w)
    worst_o = worst_l = 0.0
    for t in range(w.frames):
        if t == 14:
            gc.reset(1)
            oc.reset(1)
        for b in range(w.streams):
            gc.begin_frame(b)
            oc.begin_frame(b)
            gc.evict_frames(b)
            oc.evict(b)
        tg = gc.build_visible_page_table()
        to = oc.build_table()
        for key in ("qo_indptr", "patch_indptr", "patch_ids", "special_indptr",
                    "special_ids", "special_last_len"):
            assert np.array_equal(tg[key], getattr(to, key)), (t, key)
        gc.plan()
        # stream 1's second video draws its inputs from another seed
        qkv = [wl.frame_qkv_tensors(w, b, t, 0, seed=w.seed + (100 if b == 1 and t >= 14 else 0))
               for b in range(w.streams)]
        q, k, v = (torch.cat([x[i] for x in qkv]) for i in range(3))
        gc.append_frames(0, k.cuda(), v.cuda())
        for b in range(w.streams):
            oc.append_frame(0, b, wl.as_numpy(qkv[b][1]), wl.as_numpy(qkv[b][2]))
        o, lse = gc.attention(0, q.cuda())
        o_ref, lse_ref = paged_attention(oc.patch_pool[0], oc.special_pool[0], to,
                                         wl.as_numpy(q))
        torch.cuda.synchronize()
        worst_o = max(worst_o, float(np.abs(wl.bf16_bits_to_f32(
            o.cpu().view(torch.int16).numpy().view(np.uint16)) - o_ref).max()))
        worst_l = max(worst_l, float(np.abs(lse.cpu().numpy() - lse_ref).max()))
    gc.close()
    print("worst o", worst_o, "lse", worst_l, flush=True)
    assert worst_o <= BF16_TOL_O and worst_l <= BF16_TOL_LSE
