"""Host side of the C ABI, on the CPU (no device work).

* The built library loads and exports every symbol include/psw.h declares.
* The C++ bookkeeping matches the oracle bit for bit: page tables, free
  lists and stats after every step of random operation sequences and of the
  workloads' own sequences.
* Error paths return the documented codes and leave the state unchanged.
"""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads as wl
from oracle.cache import OracleCache
from oracle.pages import PageError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from paged_sliding_window_append_amd import _lib
    return _lib.load()


def _header_symbols():
    with open(os.path.join(ROOT, "include", "psw.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(psw_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    from paged_sliding_window_append_amd import _lib
    syms = _header_symbols()
    assert len(syms) >= 20
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(_lib.SIGNATURES)


def test_load_first_maps_one_hip_runtime():
    """Loading the library before torch must still leave one HIP runtime in
    the process (two runtimes made the library's device queries fail)."""
    import subprocess
    import sys
    code = ("import paged_sliding_window_append_amd as p; p.load(); import torch; "
            "maps = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True,
                         capture_output=True, text=True).stdout
    assert out.strip().splitlines()[-1] == "1"


def _host_cache(w, **kw):
    from paged_sliding_window_append_amd import Cache
    return Cache.for_workload(w, device=None, **kw)


def _tables_equal(t_c, t_o):
    for key in ("qo_indptr", "patch_indptr", "patch_ids", "special_indptr",
                "special_ids", "special_last_len", "special_head_len",
                "special_tail_first", "special_tail_len"):
        a = np.asarray(t_c[key])
        b = np.asarray(getattr(t_o, key))
        assert a.dtype == np.int32 and np.array_equal(a, b), key


def _compare_state(c, o, B):
    for b in range(B):
        assert c.stats(b) == o.stats(b)
        assert c.free_list(b) == o.free_list(b)


def test_stats_worked_example_via_capi():
    w = wl.MAIN.replace(max_patch_pages=88)
    c = _host_cache(w)
    for _ in range(12):
        c.begin_frame(0)
        c.evict_frames(0)
    assert c.stats(0) == {"frame_count": 12, "scale_pages": 8,
                          "live_pages": 4, "free_pages": 76,
                          "special_tokens": 72}


@pytest.mark.parametrize("name,switches", [
    ("tiny", {}), ("main_224", {}), ("keyframe_224", {}), ("interval_224", {}),
    ("large_518x378", {}),
    ("main_224", {"cross_frame_special": False}),
    ("keyframe_224", {"cross_frame_special": False}),
    ("main_224", {"include_scale_frames": False}),
    ("tiny", {"include_scale_frames": False, "cross_frame_special": False}),
])
def test_workload_sequences_match_oracle(name, switches):
    w = wl.ALL[name].replace(**switches)
    frames = min(w.frames, 400)
    c = _host_cache(w)
    o = OracleCache.for_workload(w)
    kf = [wl.keyframe_mask(w, b) for b in range(w.streams)] \
        if w.has_keyframes else None
    for t in range(frames):
        for b in range(w.streams):
            if kf is not None:
                c.set_defer_eviction(b, True)
                o.set_defer(b, True)
            c.begin_frame(b)
            o.begin_frame(b)
            c.evict_frames(b)
            o.evict(b)
        t_c = c.build_visible_page_table()
        _tables_equal(t_c, o.build_table())
        _assert_special_runs(t_c, w.special_page)
        if kf is not None:
            for b in range(w.streams):
                if kf[b][t]:
                    c.execute_deferred_eviction(b)
                    o.execute_deferred_eviction(b)
                else:
                    c.rollback_last_frame(b)
                    o.rollback_last_frame(b)
                c.set_defer_eviction(b, False)
                o.set_defer(b, False)
        _compare_state(c, o, w.streams)


def test_fixed_interval_via_capi():
    """Keyframe interval 4 over 200 frames through the C ABI: 50 frames kept
    and 300 special tokens (fixture of the 200-frame example), table and
    free list equal to the oracle's after every frame (checked above)."""
    import json
    with open(os.path.join(ROOT, "tests", "golden", "fixed_interval.json")) as f:
        g = json.load(f)
    w = wl.INTERVAL
    assert (w.frames, w.keyframe_interval) == (g["config"]["frames"],
                                               g["config"]["keyframe_interval"])
    c = _host_cache(w)
    kf = wl.keyframe_mask(w)
    for t in range(w.frames):
        c.set_defer_eviction(0, True)
        c.begin_frame(0)
        c.evict_frames(0)
        if kf[t]:
            c.execute_deferred_eviction(0)
        else:
            c.rollback_last_frame(0)
        c.set_defer_eviction(0, False)
    st_ = c.stats(0)
    assert st_["frame_count"] == g["expected"]["kept_frames"]
    assert st_["special_tokens"] == g["expected"]["special_tokens"]


OPS = ["frame", "defer_commit", "defer_rollback", "rollback", "reset",
       "evict", "defer_on", "defer_off", "begin", "chunk2", "chunk3"]


@settings(max_examples=160, deadline=None)
@given(S=st.integers(0, 3), W=st.integers(0, 4), Ns=st.integers(1, 3),
       P=st.integers(1, 4), Ps=st.integers(1, 5), extra=st.integers(0, 2),
       smax=st.integers(1, 6), B=st.integers(1, 3), isf=st.booleans(),
       cfs=st.booleans(),
       seq=st.lists(st.tuples(st.sampled_from(OPS), st.integers(0, 2)),
                    min_size=1, max_size=50))
def test_random_sequences_match_oracle(S, W, Ns, P, Ps, extra, smax, B, isf, cfs,
                                       seq):
    """Any sequence of calls, including failing ones, with or without scale
    frames and cross-frame specials: same status, same state, same table as
    the oracle."""
    from paged_sliding_window_append_amd import Cache, PswError
    if W == 0 and not cfs and (S == 0 or not isf):
        return   # nothing would be visible: refused (see test_config_rejected)
    kw = dict(layers=1, streams=B, heads=1, head_dim=64, tokens_per_frame=P + Ns,
              num_special=Ns, special_page=Ps, scale_frames=S, sliding_window=W,
              include_scale_frames=isf, cross_frame_special=cfs)
    c = Cache(dtype="fp32", max_patch_pages=S + W + 1 + extra,
              max_special_pages=smax, max_frames_per_step=3, device=None, **kw)
    o = OracleCache(pmax=S + W + 1 + extra, smax=smax, storage=np.float32, **kw)

    def both(fc, fo):
        err_c = err_o = None
        try:
            fc()
        except PswError as e:
            err_c = e.status
        try:
            fo()
        except PageError as e:
            err_o = e.code
        assert err_c == err_o

    for op, b in seq:
        b = b % B
        if op in ("frame", "begin"):
            both(lambda: c.begin_frame(b), lambda: o.begin_frame(b))
            if op == "frame":
                both(lambda: c.evict_frames(b), lambda: o.evict(b))
        elif op in ("chunk2", "chunk3"):   # joint prefill of 2 or 3 frames
            n = int(op[-1])
            both(lambda: c.begin_frames(b, n), lambda: o.begin_frames(b, n))
            both(lambda: c.evict_frames(b), lambda: o.evict(b))
        elif op == "evict":
            both(lambda: c.evict_frames(b), lambda: o.evict(b))
        elif op == "defer_on":
            c.set_defer_eviction(b, True)
            o.set_defer(b, True)
        elif op == "defer_off":
            c.set_defer_eviction(b, False)
            o.set_defer(b, False)
        elif op in ("defer_commit", "defer_rollback"):
            c.set_defer_eviction(b, True)
            o.set_defer(b, True)
            both(lambda: c.begin_frame(b), lambda: o.begin_frame(b))
            both(lambda: c.evict_frames(b), lambda: o.evict(b))
            if op == "defer_commit":
                both(lambda: c.execute_deferred_eviction(b),
                     lambda: o.execute_deferred_eviction(b))
            else:
                both(lambda: c.rollback_last_frame(b),
                     lambda: o.rollback_last_frame(b))
            c.set_defer_eviction(b, False)
            o.set_defer(b, False)
        elif op == "rollback":
            both(lambda: c.rollback_last_frame(b),
                 lambda: o.rollback_last_frame(b))
        elif op == "reset":
            c.reset(b)
            o.reset(b)
        _compare_state(c, o, B)
        t = c.build_visible_page_table()
        _tables_equal(t, o.build_table())
        _assert_special_runs(t, Ps)


def _assert_special_runs(t, Ps):
    """Each stream's listed special pages are a head run and a tail run of
    consecutive page ids: the special pool is append-only and a rollback pops
    its top, so the visible specials of the scale frames (or of every frame,
    with cross-frame specials) and of the window frames are each contiguous in
    it.  psw_plan relies on this to give the pages as two base ids when the
    list would not fit the one-launch kernel's arguments (and checks it)."""
    ind, ids = np.asarray(t["special_indptr"]), np.asarray(t["special_ids"])
    for b in range(len(ind) - 1):
        run = ids[ind[b]:ind[b + 1]]
        hp = min(len(run), -(-int(t["special_head_len"][b]) // Ps))
        for part in (run[:hp], run[hp:]):
            assert np.array_equal(part, part[:1] + np.arange(len(part))), (b, run, hp)


def test_error_codes_and_strong_guarantee():
    from paged_sliding_window_append_amd import Cache, PswError
    from paged_sliding_window_append_amd._lib import STATUS_NAMES
    c = Cache(layers=1, streams=1, heads=1, head_dim=64, dtype="bf16",
              tokens_per_frame=5, num_special=2, special_page=4,
              scale_frames=1, sliding_window=1, max_patch_pages=3,
              max_special_pages=2, device=None)
    with pytest.raises(PswError) as e:
        c.rollback_last_frame(0)
    assert STATUS_NAMES[e.value.status] == "PSW_ESTATE"
    c.begin_frame(0); c.evict_frames(0)
    c.begin_frame(0); c.evict_frames(0)
    c.set_defer_eviction(0, True)
    c.begin_frame(0); c.evict_frames(0)
    before = (c.stats(0), c.free_list(0))
    with pytest.raises(PswError) as e:
        c.begin_frame(0)
    assert STATUS_NAMES[e.value.status] == "PSW_ENOPAGE"
    assert (c.stats(0), c.free_list(0)) == before
    c.rollback_last_frame(0)
    c.begin_frame(0)                       # 3 frames = 6 specials of 8 slots
    c.rollback_last_frame(0)
    c.set_defer_eviction(0, False)
    c.begin_frame(0); c.evict_frames(0)    # 3rd frame kept: 6 specials
    c.begin_frame(0); c.evict_frames(0)    # 4th frame: 8 specials
    with pytest.raises(PswError) as e:
        c.begin_frame(0)
    assert STATUS_NAMES[e.value.status] == "PSW_ESPECIAL_FULL"
    for bad in (lambda: c.begin_frame(1), lambda: c.evict_frames(-1),
                lambda: c.stats(5)):
        with pytest.raises(PswError) as e:
            bad()
        assert STATUS_NAMES[e.value.status] == "PSW_EINVAL"
    # device calls without pools or workspace: the plan needs no workspace
    # (it asks the device for its CU count: EHIP on a host without a GPU),
    # the attention needs pools and a workspace
    c.build_visible_page_table()
    try:
        c.plan()
        planned = True
    except PswError as e:
        assert STATUS_NAMES[e.status] == "PSW_EHIP"
        planned = False
    st = c.lib.psw_attention(c.h, 0, None, None, None, None)
    assert STATUS_NAMES[st] == ("PSW_EUNBOUND" if planned else "PSW_ESTATE")
    st = c.lib.psw_append_attention_noalloc(c.h, 0, None, None, None, None, None, None)
    assert STATUS_NAMES[st] == ("PSW_EUNBOUND" if planned else "PSW_ESTATE")
    c.build_visible_page_table()   # drops the plan
    # the one-launch append + attention and its query need a plan first;
    # a failing call leaves the bookkeeping as it was
    before = (c.stats(0), c.free_list(0))
    fused = ctypes.c_int32(-1)
    assert STATUS_NAMES[c.lib.psw_plan_fused(c.h, ctypes.byref(fused))] == "PSW_ESTATE"
    assert fused.value == -1
    assert STATUS_NAMES[c.lib.psw_append_attention(c.h, 0, None, None, None, None, None,
                                                   None)] == "PSW_ESTATE"
    assert STATUS_NAMES[c.lib.psw_plan_fused(c.h, None)] == "PSW_EINVAL"
    assert STATUS_NAMES[c.lib.psw_append_attention(c.h, 3, None, None, None, None, None,
                                                   None)] == "PSW_EINVAL"
    assert (c.stats(0), c.free_list(0)) == before


@pytest.mark.parametrize("field,value", [
    ("head_dim", 128), ("num_special_tokens", 0), ("tokens_per_frame", 6),
    ("max_patch_pages", 72), ("include_scale_frames", 2),
    ("cross_frame_special", 2), ("dtype", 7), ("special_page_size", 0),
    ("sliding_window", -1), ("num_streams", 0), ("max_kv_splits", -2), ("max_kv_splits", 65),
    ("max_frames_per_step", -1), ("max_frames_per_step", 65),
])
def test_config_rejected(lib, field, value):
    from paged_sliding_window_append_amd._lib import Config
    cfg = Config(1, 1, 16, 64, 0, 262, 6, 16, 8, 64, 1, 1, 73, 120, 0, 0.0)
    assert lib.psw_config_check(ctypes.byref(cfg)) == 0
    setattr(cfg, field, value)
    assert lib.psw_config_check(ctypes.byref(cfg)) == -1
    assert lib.psw_last_error()


def test_config_nothing_visible_rejected(lib):
    """No scale frames, no window and no cross-frame specials: a frame would
    see nothing."""
    from paged_sliding_window_append_amd._lib import Config
    ok = Config(1, 1, 16, 64, 0, 262, 6, 16, 0, 64, 1, 0, 73, 120, 0, 0.0)
    assert lib.psw_config_check(ctypes.byref(ok)) == 0
    bad = Config(1, 1, 16, 64, 0, 262, 6, 16, 8, 0, 0, 0, 73, 120, 0, 0.0)
    assert lib.psw_config_check(ctypes.byref(bad)) == -1


@pytest.mark.parametrize("streams,field,value,ok", [
    # P = 262 - 6 = 256: K and V rows 2 * B * pages * 256 must stay below 2^29
    (1, "max_patch_pages", (1 << 20) - 1, True), (1, "max_patch_pages", 1 << 20, False),
    # Ps = 16: 2 * B * pages * 16 (32 streams, so the visible-token limit of
    # 2^24 per stream does not trip first)
    (32, "max_special_pages", (1 << 19) - 1, True), (32, "max_special_pages", 1 << 19, False),
])
def test_config_pool_row_limit(lib, streams, field, value, ok):
    from paged_sliding_window_append_amd._lib import Config
    cfg = Config(1, streams, 16, 64, 0, 262, 6, 16, 8, 64, 1, 1, 73, 120, 0, 0.0)
    setattr(cfg, field, value)
    assert (lib.psw_config_check(ctypes.byref(cfg)) == 0) == ok
    if not ok:
        assert b"2^29" in lib.psw_last_error()


def test_pool_bytes_layout(lib):
    from paged_sliding_window_append_amd._lib import Config
    cfg = Config(1, 4, 16, 64, 0, 1005, 6, 16, 8, 64, 1, 1, 73, 75, 0, 0.0)
    p, s, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.psw_pool_bytes(ctypes.byref(cfg), ctypes.byref(p),
                              ctypes.byref(s), ctypes.byref(w)) == 0
    assert p.value == 4 * 73 * 2 * 999 * 16 * 64 * 2
    assert s.value == 4 * 75 * 2 * 16 * 16 * 64 * 2
    # split partials at the default cap of 64: fp16 output rows (128 B) and
    # 16-byte (m, l, scale) records per (split, row, head)
    assert w.value % 256 == 0 and w.value > 64 * 4020 * 16 * (64 * 2 + 16)


def test_set_page_table_validation():
    from paged_sliding_window_append_amd import Cache, PswError
    w = wl.TINY.replace(streams=2)
    c = _host_cache(w)
    for b in range(2):
        c.begin_frame(b)
        c.evict_frames(b)
    t = c.build_visible_page_table()
    c.set_page_table(t)
    assert all(np.array_equal(c.page_table()[k], t[k]) for k in t)
    bad = dict(t)
    bad["patch_ids"] = t["patch_ids"].copy()
    bad["patch_ids"][0] = w.pmax            # belongs to stream 1
    with pytest.raises(PswError):
        c.set_page_table(bad)
    bad = dict(t)
    bad["special_last_len"] = np.array([0, 6], np.int32)
    with pytest.raises(PswError):
        c.set_page_table(bad)
    assert all(np.array_equal(c.page_table()[k], t[k]) for k in t)


def test_joint_prefill_bookkeeping():
    """A chunk of S frames at the start: the same state as S single frames,
    one table with S*T query rows, exact undo by rollback, and the limits."""
    from paged_sliding_window_append_amd import PswError
    w = wl.MAIN
    c = _host_cache(w, max_frames_per_step=w.scale_frames)
    o = OracleCache.for_workload(w)
    before = (c.stats(0), c.free_list(0))
    c.begin_frames(0, w.scale_frames)
    o.begin_frames(0, w.scale_frames)
    c.evict_frames(0)
    o.evict(0)
    t = c.build_visible_page_table()
    _tables_equal(t, o.build_table())
    assert t["qo_indptr"][1] == w.scale_frames * w.tokens_per_frame
    assert c.stats(0) == {"frame_count": 8, "scale_pages": 8, "live_pages": 0,
                          "free_pages": w.pmax - 8, "special_tokens": 48}
    c.rollback_last_frame(0)
    assert (c.stats(0), c.free_list(0)) == before
    with pytest.raises(PswError):            # above max_frames_per_step
        c.begin_frames(0, w.scale_frames + 1)
    c2 = _host_cache(w.replace(scale_frames=1, sliding_window=2),
                     max_frames_per_step=4)
    with pytest.raises(PswError):            # 3 window frames, W = 2
        c2.begin_frames(0, 4)
    c2.begin_frames(0, 3)                     # 1 scale + 2 window frames
    assert c2.stats(0)["live_pages"] == 2


def test_chunk_tables_and_workspace(lib):
    """Query rows of a custom table may be k*T up to max_frames_per_step;
    the workspace grows with it; the dense calls need a plan."""
    from paged_sliding_window_append_amd import PswError
    from paged_sliding_window_append_amd._lib import STATUS_NAMES, Config
    w = wl.TINY
    c = _host_cache(w, max_frames_per_step=2)
    c.begin_frames(0, 2)
    c.evict_frames(0)
    t = c.build_visible_page_table()
    assert t["qo_indptr"][1] == 2 * w.tokens_per_frame
    c.set_page_table(t)                       # 2T rows: accepted
    for rows in (3 * w.tokens_per_frame, w.tokens_per_frame + 1):
        bad = dict(t)
        bad["qo_indptr"] = np.array([0, rows], np.int32)
        with pytest.raises(PswError) as e:
            c.set_page_table(bad)
        assert STATUS_NAMES[e.value.status] == "PSW_EINVAL"
    with pytest.raises(PswError) as e:
        c.visible_tokens()                    # no plan yet
    assert STATUS_NAMES[e.value.status] == "PSW_ESTATE"
    ws = []
    for f in (0, 1, 8):
        cfg = Config(1, 1, 16, 64, 0, 262, 6, 16, 8, 64, 1, 1, 73, 120, 0, 0.0, f)
        p_, s_, w_ = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.psw_pool_bytes(ctypes.byref(cfg), ctypes.byref(p_), ctypes.byref(s_),
                                  ctypes.byref(w_)) == 0
        ws.append(w_.value)
    assert ws[0] == ws[1] < ws[2]


def test_shared_head_tail_page_round_trip():
    """Without cross-frame specials the head range (scale frames) and the
    tail range (window frames) can start and end in the same special page,
    which the table then lists twice: max_special_pages + 1 entries.  The
    table read back must be accepted again as it is."""
    from paged_sliding_window_append_amd import Cache
    c = Cache(layers=1, streams=1, heads=1, head_dim=64, dtype="bf16",
              tokens_per_frame=22, num_special=6, special_page=16,
              scale_frames=1, sliding_window=1, max_patch_pages=3,
              max_special_pages=2, cross_frame_special=False, device=None)
    seen_shared = False
    for _ in range(3):
        c.begin_frame(0)
        c.evict_frames(0)
        tb = c.build_visible_page_table()
        seen_shared |= len(tb["special_ids"]) == 3
        c.set_page_table(tb)
        back = c.page_table()
        for key, val in tb.items():
            assert np.array_equal(back[key], val), key
    assert seen_shared


def test_profile_calls_on_the_host(lib):
    """Timing calls without any launch: enabling and reading work on a cache
    that never touches a device (no events, zero sums and counts); a NULL
    cache is refused."""
    from paged_sliding_window_append_amd import Cache
    c = Cache(layers=1, streams=1, heads=1, head_dim=64, dtype="bf16",
              tokens_per_frame=5, num_special=2, special_page=4,
              scale_frames=1, sliding_window=1, max_patch_pages=3,
              max_special_pages=2, device=None)
    a, m = ctypes.c_double(-1.0), ctypes.c_double(-1.0)
    na, nm = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert lib.psw_profile_enable(c.h, 1) == 0
    assert lib.psw_profile_read(c.h, ctypes.byref(a), ctypes.byref(na),
                                ctypes.byref(m), ctypes.byref(nm)) == 0
    assert (a.value, na.value, m.value, nm.value) == (0.0, 0, 0.0, 0)
    assert lib.psw_profile_enable(c.h, 0) == 0
    assert lib.psw_profile_enable(None, 1) != 0
    assert lib.psw_profile_read(None, None, None, None, None) != 0
    c.close()


def test_bind_validation(lib):
    """Pools and workspace are validated when bound (no device access):
    NULL, misaligned, a layer out of range and a workspace smaller than
    psw_pool_bytes reports are refused with PSW_EINVAL; fitting ones bind.
    The addresses are never dereferenced by these calls."""
    from paged_sliding_window_append_amd import Cache
    from paged_sliding_window_append_amd._lib import STATUS_NAMES
    c = Cache(layers=2, streams=1, heads=1, head_dim=64, dtype="bf16",
              tokens_per_frame=5, num_special=2, special_page=4,
              scale_frames=1, sliding_window=1, max_patch_pages=3,
              max_special_pages=2, device=None)
    pb, sb, wb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.psw_pool_bytes(ctypes.byref(c.cfg), ctypes.byref(pb), ctypes.byref(sb),
                              ctypes.byref(wb)) == 0
    a16, a256 = 1 << 20, 1 << 20   # aligned stand-in addresses
    name = lambda st: STATUS_NAMES[st]  # noqa: E731
    assert name(lib.psw_bind_layer(c.h, 0, None, a16)) == "PSW_EINVAL"
    assert name(lib.psw_bind_layer(c.h, 0, a16 + 8, a16)) == "PSW_EINVAL"
    assert name(lib.psw_bind_layer(c.h, 2, a16, a16)) == "PSW_EINVAL"
    assert name(lib.psw_bind_layer(c.h, 1, a16, a16)) == "PSW_OK"
    assert name(lib.psw_bind_workspace(c.h, None, wb.value)) == "PSW_EINVAL"
    assert name(lib.psw_bind_workspace(c.h, a256 + 16, wb.value)) == "PSW_EINVAL"
    assert name(lib.psw_bind_workspace(c.h, a256, wb.value - 1)) == "PSW_EINVAL"
    assert name(lib.psw_bind_workspace(c.h, a256, wb.value)) == "PSW_OK"
    c.close()
