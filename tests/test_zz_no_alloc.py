"""psw_append_attention_noalloc (the entry point that allocates nothing: its
workspace is the library's static scratch array) against
psw_append_attention, through the C ABI.

Twin caches get the same calls and inputs; the one using the no-alloc entry
point has no workspace bound at all.  Output, log-sum-exp and pool bytes must
be bit-identical (the same kernels run on the same plan; only where the
plan and the split partials live differs), and the result must match the
oracle within the bf16 tolerances.  Three workloads in a row, the last the
smallest, so each after the first reuses a scratch array that the one before
left full of its own plan and partials; the second has plans that give the
special pages as two runs of page ids."""
import numpy as np
import pytest

import workloads as wl
from _parity import BF16_TOL_LSE, BF16_TOL_O, pool_bytes, to_np
from oracle.attention import paged_attention
from oracle.cache import OracleCache

pytestmark = pytest.mark.gpu


def _twins(w, frames_checked, fused_from=None):
    import torch
    from paged_sliding_window_append_amd import Cache
    ref = Cache.for_workload(w)
    na = Cache.for_workload(w, workspace=False)
    oc = OracleCache.for_workload(w)
    rows = w.streams * w.tokens_per_frame
    o = [torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
         for _ in range(2)]
    lse = [torch.empty((rows, w.heads), dtype=torch.float32, device="cuda")
           for _ in range(2)]
    worst_o = worst_lse = 0.0
    identical = 0
    for t in range(w.frames):
        for c in (ref, na):
            for b in range(w.streams):
                c.begin_frame(b)
                c.evict_frames(b)
            c.build_visible_page_table()
            c.plan()
        for b in range(w.streams):
            oc.begin_frame(b)
            oc.evict(b)
        to = oc.build_table()
        qkv = [wl.frame_qkv_tensors(w, b, t, 0) for b in range(w.streams)]
        q, k, v = (torch.cat([x[i] for x in qkv]).cuda() for i in range(3))
        for b in range(w.streams):
            oc.append_frame(0, b, wl.as_numpy(qkv[b][1]), wl.as_numpy(qkv[b][2]))
        if fused_from is not None and t >= fused_from:
            assert na.plan_fused(), f"one launch, frame {t}"
        ref.append_attention(0, k, v, q, o[0], lse[0])
        na.append_attention(0, k, v, q, o[1], lse[1], noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(o[0].view(torch.int16), o[1].view(torch.int16)), f"o, frame {t}"
        assert torch.equal(lse[0], lse[1]), f"lse, frame {t}"
        identical += 1
        if t in frames_checked:
            o_ref, lse_ref = paged_attention(oc.patch_pool[0], oc.special_pool[0], to,
                                             wl.as_numpy(q.cpu()))
            worst_o = max(worst_o, float(np.abs(to_np(o[1]) - o_ref).max()))
            worst_lse = max(worst_lse, float(np.abs(to_np(lse[1]) - lse_ref).max()))
    for a, b in ((ref.patch_pools[0], na.patch_pools[0]),
                 (ref.special_pools[0], na.special_pools[0])):
        assert np.array_equal(pool_bytes(a), pool_bytes(b))
    assert np.array_equal(pool_bytes(na.patch_pools[0]), oc.patch_pool[0])
    assert np.array_equal(pool_bytes(na.special_pools[0]), oc.special_pool[0])
    items, splits = na.plan_info()
    ref.close()
    na.close()
    print(f"{w.name}: {identical} frames bit-identical, last plan {items} items, "
          f"{splits} splits; oracle o {worst_o:.3g} lse {worst_lse:.3g}", flush=True)
    assert worst_o <= BF16_TOL_O and worst_lse <= BF16_TOL_LSE
    return splits


def test_noalloc_matches_workspace_entry_point(gpu):
    # first: the 262 tok/frame geometry through the window filling (16 KV
    # splits at the end); then 25 specials a frame on 2-token pages without
    # cross-frame specials (from about frame 51 the listed special pages keep
    # the list out of the one-launch kernel's arguments: the plan gives them as
    # runs); then a smaller ragged batch of three streams
    big = wl.MAIN.replace(frames=76)
    s1 = _twins(big, {0, 8, 72, 75})
    assert s1 > 1
    runs = wl.Workload("noalloc_runs", layers=1, heads=16, head_dim=64, dtype="bf16",
                       tokens_per_frame=262, num_special=25, special_page=2,
                       scale_frames=8, sliding_window=72, frames=90, streams=1,
                       cross_frame_special=False, seed=4)
    _twins(runs, {60, 89}, fused_from=0)
    small = wl.Workload("noalloc_small", layers=1, heads=3, head_dim=64, dtype="bf16",
                        tokens_per_frame=70, num_special=5, special_page=3,
                        scale_frames=1, sliding_window=3, frames=12, streams=3, seed=9)
    _twins(small, {0, 5, 11})
