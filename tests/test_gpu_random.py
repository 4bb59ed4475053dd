"""GPU parity on seeded random geometries: the HIP path through the C ABI
against the oracle, every frame, with tables, free lists and pool bytes
bit-exact and attention within the bf16 tolerances; the random draws mix
streams, page sizes, windows, both switches, keyframe masks, a joint first
chunk and the dense float32 check path."""
import numpy as np
import pytest

import workloads as wl
from _parity import BF16_TOL_LSE, BF16_TOL_O, run
from test_gpu_parity import _ok_bf16

pytestmark = pytest.mark.gpu


def _draw(seed):
    r = np.random.default_rng(seed)
    while True:
        Ns = int(r.integers(1, 9))
        g = dict(tokens_per_frame=Ns + int(r.integers(1, 300)), num_special=Ns,
                 special_page=int(r.integers(1, 21)), scale_frames=int(r.integers(0, 5)),
                 sliding_window=int(r.integers(0, 7)), heads=int(r.integers(1, 5)),
                 frames=int(r.integers(3, 16)), streams=int(r.integers(1, 4)),
                 include_scale_frames=bool(r.integers(0, 2)),
                 cross_frame_special=bool(r.integers(0, 2)))
        S = g["scale_frames"] if g["include_scale_frames"] else 0
        if S == 0 and g["sliding_window"] == 0 and not g["cross_frame_special"]:
            continue   # nothing would be visible: refused
        # even seeds: a joint first chunk; odd seeds: keyframe masks
        chunk, kfp = 1, None
        if seed % 2 == 0:
            top = min(g["frames"], S + g["sliding_window"])
            if top < 2:
                continue
            chunk = int(r.integers(2, top + 1))
        else:
            kfp = 0.5
        return g, chunk, kfp


@pytest.mark.parametrize("seed", range(10))
def test_random_geometry_every_frame(gpu, seed):
    g, chunk, kfp = _draw(1000 + seed)
    w = wl.Workload(f"rand{seed}", layers=1, head_dim=64, dtype="bf16", seed=seed,
                    keyframe_p=kfp, **g)
    kf = None if kfp is None else [wl.keyframe_mask(w, b) for b in range(w.streams)]
    print(g, "chunk", chunk, "keyframes", kfp is not None, flush=True)
    worst = run(w, keyframes=kf, first_chunk=chunk, pools_at=[w.frames - 1],
                dense_at={w.frames - 1}, cache_kw={"max_frames_per_step": max(chunk, 1)})
    _ok_bf16(worst)
    assert worst.cross_o <= BF16_TOL_O and worst.cross_lse <= BF16_TOL_LSE
