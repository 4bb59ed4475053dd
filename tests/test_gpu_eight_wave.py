"""The 8-wave attention shape on work items of one to three key tiles.

The plan takes 8-wave workgroups when the frame is large (one workgroup per
compute unit, half the KV splits); their waves 4..7 run each fast key tile
half a tile behind waves 0..3, with the second half's scores and V fragments
carried in registers across the tile's barrier.  On the full-size workloads
every 8-wave work item spans several key tiles; here a second stream that
keeps none of its frames (no scale frames, no window kept: every frame is
rolled back after its attention) sees only its current frame, one to three
key tiles with a partial last one, inside the same 8-wave launch as a stream
whose window has grown to ~100 tiles.  Token-exact inputs
(``workloads.frame_qkv_coded``): a dropped, repeated or misplaced key shows
in the log-sum-exp or the per-class counts.
"""
import numpy as np
import pytest

import workloads as wl
from _parity import run
from test_gpu_exact import _ok_exact

pytestmark = pytest.mark.gpu


# tokens per frame (the short stream's keys: 1, 2 and 3 key tiles), window and
# frames so that the long stream passes the ~32 key tiles where 8 waves start
# (the 8-wave shape then runs from frame 32, 19 and 12 on)
@pytest.mark.parametrize("T,window,frames", [(60, 96, 110), (100, 64, 72), (150, 64, 52)])
def test_eight_wave_short_items_exact(gpu, T, window, frames):
    w = wl.Workload(f"eight_wave_{T}", layers=1, heads=16, head_dim=64, dtype="bf16",
                    tokens_per_frame=T, num_special=6, special_page=16, scale_frames=0,
                    sliding_window=window, frames=frames, streams=2,
                    include_scale_frames=False, cross_frame_special=False, seed=T)
    keep = [np.ones(frames, dtype=bool), np.zeros(frames, dtype=bool)]
    waves = {}
    worst = run(w, keyframes=keep, exact=True, fused=True,
                on_plan=lambda t, c: waves.__setitem__(t, c.plan_waves()))
    eight = sorted(t for t, v in waves.items() if v == 8)
    print(f"T={T}: 8-wave frames {eight[:1]}..{eight[-1:]} ({len(eight)})", flush=True)
    _ok_exact(worst, frames)
    assert len(eight) >= 5 and eight[-1] == frames - 1
