"""GPU checks of the dense float32 path (the pages' force_fp32 mode: the
paged K/V gathered into dense tensors, attention in float for validation).

* The gathered K/V equal the oracle's gather of the visible tokens bit for
  bit (bf16 widened exactly), stream by stream.
* The dense attention matches the float64 oracle within 1e-4 (max-abs on o
  and lse).
* As a second GPU check of the paged bf16 MFMA kernel, its o/lse match the
  dense float32 result on every row and head within the bf16 tolerances
  (1e-2 on o, 1e-3 on lse) -- at full size, where the oracle is sampled.
"""
import pytest

import workloads as wl
from _parity import BF16_TOL_LSE, BF16_TOL_O, FP32_TOL, run
from test_gpu_parity import SMALL_BF16, _ok_bf16

pytestmark = pytest.mark.gpu


def _ok_dense(worst, cross=True):
    print(f"dense o {worst.dense_o:.3g} lse {worst.dense_lse:.3g}; paged vs dense "
          f"o {worst.cross_o:.3g} lse {worst.cross_lse:.3g} over "
          f"{worst.dense_checked} checks", flush=True)
    assert worst.dense_checked > 0
    assert worst.dense_o <= FP32_TOL
    assert worst.dense_lse <= FP32_TOL
    if cross:
        assert worst.cross_o <= BF16_TOL_O
        assert worst.cross_lse <= BF16_TOL_LSE


def test_dense_tiny_fp32_every_frame(gpu):
    w = wl.TINY
    worst = run(w, dense_at=range(w.frames))
    assert worst.o <= FP32_TOL and worst.lse <= FP32_TOL
    _ok_dense(worst)
    assert worst.cross_o <= FP32_TOL and worst.cross_lse <= FP32_TOL


DENSE_SMALL = [
    # (geometry, switches, keyframe probability): several 64-key tiles,
    # three ragged streams, head and tail special ranges, defer/rollback
    (1, {}, None),
    (2, {}, None),
    (5, {}, None),
    (2, {"cross_frame_special": False}, None),
    (3, {"cross_frame_special": False, "include_scale_frames": False}, None),
    (2, {"cross_frame_special": False}, 0.5),
]


@pytest.mark.parametrize("i", range(len(DENSE_SMALL)))
def test_dense_small_every_frame(gpu, i):
    g, sw, kfp = DENSE_SMALL[i]
    w = wl.Workload(f"dense{i}", layers=1, head_dim=64, dtype="bf16", seed=60 + i,
                    keyframe_p=kfp, **SMALL_BF16[g], **sw)
    kf = None if kfp is None else [wl.keyframe_mask(w, b) for b in range(w.streams)]
    worst = run(w, keyframes=kf, dense_at=range(w.frames))
    _ok_bf16(worst)
    _ok_dense(worst)


def test_dense_main_224(gpu):
    """262 tok/frame, 320 frames: the window full (frame 72) and the last
    frame, every row and head of the paged kernel against the dense path."""
    w = wl.MAIN
    worst = run(w, attend=lambda t: t in {72, 319}, dense_at={72, 319},
                heads_checked=[0, 11])
    _ok_bf16(worst)
    _ok_dense(worst)


def test_dense_large_518x378(gpu):
    """Four streams of 999 + 6 tokens at frame 79 (window full): 72 408
    visible tokens per stream (999 * 72 patches + 6 * 80 specials)."""
    w = wl.LARGE.replace(frames=80)
    worst = run(w, attend=lambda t: t == 79, dense_at={79}, heads_checked=[5])
    _ok_bf16(worst)
    _ok_dense(worst)
