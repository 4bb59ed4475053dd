"""GPU parity of the fused append + attention entry point
(psw_append_attention) against the oracle: the same workloads as the
separate calls, with tables, free lists, stats and the pool bytes the launch
writes bit-exact and attention within the bf16 tolerances (1e-2 on o, 1e-3
on lse, 2e-2 relative).  Each test also states whether the one-launch form
ran (the plan fits its kernel arguments) or the entry point made the two
calls."""
import pytest

import workloads as wl
from _parity import BF16_TOL_LSE, BF16_TOL_O, BF16_TOL_REL, FP32_TOL, run
from test_gpu_joint import JOINT_SMALL
from test_gpu_parity import SMALL_BF16, SWITCHES, _ok_bf16
from test_gpu_random import _draw

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(len(SMALL_BF16)))
def test_fused_small_every_frame(gpu, i):
    w = wl.Workload(f"fsmall{i}", layers=2, head_dim=64, dtype="bf16", seed=i,
                    **SMALL_BF16[i])
    worst = run(w, pools_at=[w.frames // 2, w.frames - 1], fused=True)
    _ok_bf16(worst)
    print("fused steps", worst.fused_steps, "of", w.frames * w.layers, flush=True)
    assert worst.fused_steps > 0


@pytest.mark.parametrize("i", range(len(SWITCHES)))
def test_fused_switches_every_frame(gpu, i):
    g, sw = SWITCHES[i]
    w = wl.Workload(f"fswitch{i}", layers=2, head_dim=64, dtype="bf16", seed=40 + i,
                    **SMALL_BF16[g], **sw)
    worst = run(w, pools_at=[w.frames - 1], fused=True)
    _ok_bf16(worst)
    print("fused steps", worst.fused_steps, "of", w.frames * w.layers, flush=True)
    assert worst.fused_steps > 0


def test_fused_keyframes_ragged(gpu):
    """Deferred eviction and rollback on three streams with their own
    keyframe masks, both special switches."""
    for cross in (True, False):
        w = wl.Workload("fragged", layers=1, heads=2, head_dim=64, dtype="bf16",
                        tokens_per_frame=70, num_special=6, special_page=16,
                        scale_frames=2, sliding_window=5, frames=40, streams=3,
                        keyframe_p=0.5, seed=11, cross_frame_special=cross)
        kf = [wl.keyframe_mask(w, b) for b in range(w.streams)]
        worst = run(w, keyframes=kf, pools_at=[w.frames - 1], fused=True)
        _ok_bf16(worst)
        print("fused steps", worst.fused_steps, "of", w.frames, flush=True)
        assert worst.fused_steps > 0


@pytest.mark.parametrize("i", range(len(JOINT_SMALL)))
def test_fused_joint_every_frame(gpu, i):
    """A joint first chunk: several current frames per stream read from k/v."""
    g, n, sw = JOINT_SMALL[i]
    w = wl.Workload(f"fjoint{i}", layers=2, head_dim=64, dtype="bf16", seed=80 + i,
                    **SMALL_BF16[g], **sw)
    worst = run(w, first_chunk=n, pools_at=[n - 1, w.frames - 1],
                cache_kw={"max_frames_per_step": n}, fused=True)
    _ok_bf16(worst)
    print("fused steps", worst.fused_steps, "of", (w.frames - n + 1) * w.layers, flush=True)
    assert worst.fused_steps > 0


@pytest.mark.parametrize("seed", range(10))
def test_fused_random_geometry_every_frame(gpu, seed):
    g, chunk, kfp = _draw(1000 + seed)
    w = wl.Workload(f"frand{seed}", layers=1, head_dim=64, dtype="bf16", seed=seed,
                    keyframe_p=kfp, **g)
    kf = None if kfp is None else [wl.keyframe_mask(w, b) for b in range(w.streams)]
    print(g, "chunk", chunk, "keyframes", kfp is not None, flush=True)
    worst = run(w, keyframes=kf, first_chunk=chunk, pools_at=[w.frames - 1],
                cache_kw={"max_frames_per_step": max(chunk, 1)}, fused=True)
    _ok_bf16(worst)
    print("fused steps", worst.fused_steps, flush=True)
    _random_fused_steps.append(worst.fused_steps)


_random_fused_steps = []


def test_fused_random_geometry_took_one_launch(gpu):
    """The random geometries above did exercise the one-launch form (each
    seed's plan may fall back to the two calls, not all of them)."""
    if len(_random_fused_steps) < 10:
        pytest.skip("run together with test_fused_random_geometry_every_frame")
    assert sum(_random_fused_steps) > 0


def test_fused_main_224_every_frame(gpu):
    """The 262 tok/frame workload: every frame in one launch, attention
    against the oracle on all 320 frames and all 16 heads."""
    w = wl.MAIN
    worst = run(w, pools_at=[71, 319], fused=True, log_every=64)
    _ok_bf16(worst)
    assert worst.checked == w.frames
    assert worst.fused_steps == w.frames


def test_fused_keyframe_224_transitions(gpu):
    """Deferred eviction and rollback through the one-launch path: attention
    against the oracle at all 126 keyframe transitions of frames 1-299, at
    frames 243-250 (the window full under deferral: W + 1 window pages
    resident, the last W visible) and at the last frame."""
    w = wl.KEYFRAME
    kf = [wl.keyframe_mask(w, 0)]
    trans = [t for t in range(1, 300) if kf[0][t] != kf[0][t - 1]]
    assert len(trans) == 126
    sample = set(trans) | set(range(243, 251)) | {0, w.frames - 1}
    worst = run(w, keyframes=kf, attend=lambda t: t in sample,
                pools_at=[w.frames - 1], fused=True, log_every=200)
    _ok_bf16(worst)
    assert worst.checked == len(sample)
    assert worst.fused_steps == w.frames


def test_fused_main_224_no_cross_frame_specials(gpu):
    w = wl.MAIN.replace(cross_frame_special=False)
    sample = {0, 71, 72, 73, 319}
    worst = run(w, attend=lambda t: t in sample, heads_checked=[0, 15],
                pools_at=[319], fused=True)
    _ok_bf16(worst)
    assert worst.fused_steps == w.frames


def test_fused_stack_224x24_sampled(gpu):
    w = wl.STACK.replace(frames=80)
    sample = {0, 71, 72, 79}
    worst = run(w, attend=lambda t: t in sample, layers_checked=[0, 23],
                pools_at=[79], fused=True)
    _ok_bf16(worst)
    assert worst.fused_steps == w.frames * w.layers


def test_fused_peaked_softmax(gpu):
    """q x 8: a peaked softmax (weights up to about 2^19 against the first
    tile's reference; the rerun of a workgroup's range is exercised by
    test_overflow_vote_reruns_exactly).  With 4 heads the later frames' plans
    outgrow the kernel arguments: those frames take the two-call form."""
    w = wl.MAIN.replace(frames=80, heads=4)
    worst = run(w, q_scale=8.0, attend=lambda t: t in (0, 5, 40, 71, 72, 79),
                fused=True)
    print("fused steps", worst.fused_steps, "of", w.frames, flush=True)
    assert worst.checked == 6 and worst.fused_steps > 0
    assert worst.scaled <= 2.0 ** -8
    assert worst.lse <= BF16_TOL_LSE
    assert worst.rel <= BF16_TOL_REL


def test_fused_falls_back(gpu):
    """Where the one-launch form does not apply the entry point makes the two
    calls: float32, a caller's (reordered) table."""
    w = wl.TINY
    worst = run(w, pools_at=[w.frames - 1], fused=True)
    assert worst.fused_steps == 0
    assert worst.o <= FP32_TOL and worst.lse <= FP32_TOL

    w = wl.TINY.replace(dtype="bf16", frames=10, heads=2, streams=2)

    def reverse(t, tbl):
        tbl = {k: v.copy() for k, v in tbl.items()}
        for b in range(2):
            s, e = tbl["patch_indptr"][b], tbl["patch_indptr"][b + 1]
            tbl["patch_ids"][s:e] = tbl["patch_ids"][s:e][::-1]
        return tbl
    worst = run(w, table_hook=reverse, fused=True)
    _ok_bf16(worst)
    assert worst.fused_steps == 0



def test_fused_large_518x378_both_forms(gpu):
    """Four 1005-token streams (four query blocks each): the early frames'
    plans fit the kernel arguments and run as one launch, the later ones
    (more pages, splits and scores) take the two-call form."""
    w = wl.LARGE.replace(frames=80)
    worst = run(w, attend=lambda t: t in (0, 9, 40, 79), heads_checked=[0, 15],
                pools_at=[9, 79], fused=True)
    _ok_bf16(worst)
    print("fused steps", worst.fused_steps, "of", w.frames, flush=True)
    assert 0 < worst.fused_steps < w.frames


def test_fused_bit_identical_to_two_calls(gpu):
    """Same plan, same arithmetic: the one launch (current frames read from
    k/v) and the two calls (read from the pool after the append kernel)
    give the same output, log-sum-exp and pool bytes, bit for bit, on every
    frame of the 224x224 workload through the window filling (90 frames,
    4 heads) and on a three-stream ragged keyframe batch."""
    import numpy as np
    import torch
    from paged_sliding_window_append_amd import Cache

    def stream(w, kf=None):
        outs = []
        caches = [Cache.for_workload(w), Cache.for_workload(w)]
        for t in range(w.frames):
            for c in caches:
                for b in range(w.streams):
                    if kf is not None:
                        c.set_defer_eviction(b, True)
                    c.begin_frame(b)
                    c.evict_frames(b)
                c.build_visible_page_table()
                c.plan()
            qkv = [wl.frame_qkv_tensors(w, b, t, 0) for b in range(w.streams)]
            q, k, v = (torch.cat([x[i] for x in qkv]).cuda() for i in range(3))
            fused = caches[0].plan_fused()
            o1, l1 = caches[0].append_attention(0, k, v, q)
            caches[1].append_frames(0, k, v)
            o2, l2 = caches[1].attention(0, q)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), t
            assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), t
            outs.append(fused)
            if kf is not None:
                for c in caches:
                    for b in range(w.streams):
                        if kf[b][t]:
                            c.execute_deferred_eviction(b)
                        else:
                            c.rollback_last_frame(b)
                        c.set_defer_eviction(b, False)
        for a, b in zip(caches[0].patch_pools + caches[0].special_pools,
                        caches[1].patch_pools + caches[1].special_pools):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        for c in caches:
            c.close()
        return outs

    fused = stream(wl.MAIN.replace(frames=90, heads=4))
    assert sum(fused) > 0
    w = wl.Workload("fbits", layers=1, heads=2, head_dim=64, dtype="bf16",
                    tokens_per_frame=70, num_special=6, special_page=16,
                    scale_frames=2, sliding_window=5, frames=30, streams=3,
                    keyframe_p=0.5, seed=13)
    fused = stream(w, [wl.keyframe_mask(w, b) for b in range(w.streams)])
    assert all(fused)


def _weights_overflow_first_tile(w, frame, q_scale):
    """Heads in which some query's weight against the first key tile's
    reference exceeds 2^64 at `frame` (one KV split per stream, so the first
    tile is the first 64 visible keys): there the fast form's running sums
    overflow its limit, and the workgroup must rerun its key range in the
    exact form.  Computed on the host from the oracle's visible keys."""
    import numpy as np
    from oracle.attention import gather_visible_kv
    from oracle.cache import OracleCache
    oc = OracleCache.for_workload(w)
    for t in range(frame + 1):
        oc.begin_frame(0)
        oc.evict(0)
        _, k, v = wl.frame_qkv(w, 0, t, 0, q_scale)
        oc.append_frame(0, 0, k, v)
    table = oc.build_table()
    kk, _ = gather_visible_kv(oc.patch_pool[0], oc.special_pool[0], table, 0)
    q, _, _ = wl.frame_qkv(w, 0, frame, 0, q_scale)
    kf = wl.bf16_bits_to_f32(kk).astype(np.float64)
    qf = wl.bf16_bits_to_f32(q).astype(np.float64)
    s = np.einsum("rhd,khd->hrk", qf, kf) / np.sqrt(w.head_dim)   # [H, rows, keys]
    excess = s.max(axis=2) - s[:, :, :64].max(axis=2)
    return [h for h in range(w.heads) if (excess[h] > 64 * np.log(2.0)).any()]


@pytest.mark.parametrize("fused", [True, False])
def test_overflow_vote_reruns_exactly(gpu, fused):
    """q x 32 with one KV split per stream: later keys' weights outgrow the
    first tile's reference by more than 2^64 (checked on the host first), so
    the end-of-loop vote sends the workgroup back over its whole key range
    in the exact form (on the one-launch path rereading the current frame
    from k/v).  The result must still match the oracle, with the bound of
    the other peaked runs."""
    w = wl.MAIN.replace(frames=80, heads=4)
    checked = (72, 79)
    for t in checked:
        heads = _weights_overflow_first_tile(w, t, 32.0)
        print("frame", t, "heads whose sums overflow the fast form:", heads, flush=True)
        assert heads, "the inputs do not overflow the fast form"
    worst = run(w, q_scale=32.0, attend=lambda t: t in checked, fused=fused,
                cache_kw={"max_kv_splits": 1})
    print(worst, flush=True)
    assert worst.checked == len(checked)
    assert worst.scaled <= 2.0 ** -8
    assert worst.lse <= BF16_TOL_LSE
    assert worst.rel <= BF16_TOL_REL
    if fused:
        assert worst.fused_steps == w.frames


def _overflowing_splits(w, frame, q_scale, ns, heads):
    """(split, head) pairs of a one-stream frame planned into `ns` KV splits
    of whole key tiles (split s starts at tile kvt * s / ns, as the plan cuts
    them) in which some query's weight against the split's first key tile
    exceeds 2^64, so that workgroup must rerun its range."""
    import numpy as np
    from oracle.attention import gather_visible_kv
    from oracle.cache import OracleCache
    oc = OracleCache.for_workload(w)
    for t in range(frame + 1):
        oc.begin_frame(0)
        oc.evict(0)
        _, k, v = wl.frame_qkv(w, 0, t, 0, q_scale)
        oc.append_frame(0, 0, k, v)
    kk, _ = gather_visible_kv(oc.patch_pool[0], oc.special_pool[0], oc.build_table(), 0)
    q, _, _ = wl.frame_qkv(w, 0, frame, 0, q_scale)
    kf = wl.bf16_bits_to_f32(kk).astype(np.float32)
    qf = wl.bf16_bits_to_f32(q).astype(np.float32)
    L = kf.shape[0]
    kvt = -(-L // 64)
    out = []
    for h in heads:
        s = (qf[:, h] @ kf[:, h].T).astype(np.float64) / np.sqrt(w.head_dim)   # [rows, keys]
        for sp in range(ns):
            k0, k1 = kvt * sp // ns * 64, min(kvt * (sp + 1) // ns * 64, L)
            excess = s[:, k0:k1].max(axis=1) - s[:, k0:k0 + 64].max(axis=1)
            if (excess > 64 * np.log(2.0)).any():
                out.append((sp, h))
    return out


@pytest.mark.parametrize("fused", [True, False])
def test_overflow_vote_reruns_exactly_eight_waves(gpu, fused):
    """The same in the 8-wave shape (16 heads, 16 KV splits at the checked
    frames, lagged waves 4-7): q x 128 makes later keys of a split outgrow
    its first tile's reference by more than 2^64 (counted on the host from
    the plan's own split count after the run)."""
    w = wl.MAIN.replace(frames=80)
    checked = (72, 79)
    heads = [0, 5, 10, 15]
    plans = {}

    def record(t, gc):
        if t in checked:
            plans[t] = (gc.plan_info(), gc.plan_waves())
    worst = run(w, q_scale=128.0, attend=lambda t: t in checked, fused=fused,
                on_plan=record, heads_checked=heads)
    print(worst, flush=True)
    for t in checked:
        (items, ns), waves = plans[t]
        assert waves == 8, (t, plans[t])
        over = _overflowing_splits(w, t, 128.0, ns, heads)
        print("frame", t, "splits", ns, "overflowing (split, head) pairs:", len(over),
              flush=True)
        assert len(over) > 0
    assert worst.checked == len(checked)
    assert worst.scaled <= 2.0 ** -8
    assert worst.lse <= BF16_TOL_LSE
    assert worst.rel <= BF16_TOL_REL
    if fused:
        assert worst.fused_steps == w.frames


@pytest.mark.parametrize("fused", [True, False])
def test_merge_of_17_to_32_splits(gpu, fused):
    """8 heads of the 224x224 geometry: once the window has filled the plan
    splits each head's keys 17 to 32 ways (8-wave workgroups), the range the
    merge kernel serves with 8 split groups of up to 4 splits per lane."""
    w = wl.MAIN.replace(frames=80, heads=8)
    checked = (40, 72, 79)
    splits = {}

    def record(t, gc):
        if t in checked:
            splits[t] = gc.plan_info()[1]
    worst = run(w, attend=lambda t: t in checked, fused=fused, on_plan=record)
    print(worst, splits, flush=True)
    assert all(17 <= splits[t] <= 32 for t in (72, 79)), splits
    _ok_bf16(worst)
    assert worst.checked == len(checked)


def test_profile_counts_launches(gpu):
    """Kernel timing: while enabled, every attention launch and every merge
    launch gets an event pair; a read returns positive summed durations and
    the launch counts and clears them; while disabled nothing is recorded."""
    import ctypes
    import torch
    from paged_sliding_window_append_amd import Cache
    w = wl.MAIN.replace(frames=20, heads=4)
    c = Cache.for_workload(w, device="cuda:0")
    lib, h = c.lib, c.h

    def read():
        a, m = ctypes.c_double(), ctypes.c_double()
        na, nm = ctypes.c_int32(), ctypes.c_int32()
        assert lib.psw_profile_read(h, ctypes.byref(a), ctypes.byref(na),
                                    ctypes.byref(m), ctypes.byref(nm)) == 0
        return a.value, na.value, m.value, nm.value
    merges = 0
    for t in range(w.frames):
        lib.psw_profile_enable(h, int(t % 2 == 0))
        c.begin_frame(0)
        c.evict_frames(0)
        c.build_visible_page_table()
        c.plan()
        q, k, v = wl.frame_qkv_tensors(w, 0, t, 0)
        c.append_attention(0, k.cuda(), v.cuda(), q.cuda())
        merges += int(t % 2 == 0 and c.plan_info()[1] > 1)
    torch.cuda.synchronize()
    a, na, m, nm = read()
    print("attention", a, na, "merge", m, nm, flush=True)
    assert na == w.frames // 2 and a > 0.0
    assert nm == merges and (m > 0.0) == (merges > 0)
    assert read() == (0.0, 0, 0.0, 0)          # cleared by the read
    lib.psw_profile_enable(h, 0)
    c.begin_frame(0)
    c.evict_frames(0)
    c.build_visible_page_table()
    c.plan()
    q, k, v = wl.frame_qkv_tensors(w, 0, w.frames, 0)
    c.append_attention(0, k.cuda(), v.cuda(), q.cuda())
    torch.cuda.synchronize()
    assert read() == (0.0, 0, 0.0, 0)          # nothing while disabled
    c.close()
