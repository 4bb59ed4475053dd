"""GPU parity of joint prefill: the first frames begun, written and attended
as one chunk (every query of the chunk sees all of its frames), then single
frames -- the HIP path through the C ABI against the oracle, with the bf16
tolerances (1e-2 on o, 1e-3 on lse, 2e-2 relative), tables, free lists and
pool bytes bit-exact."""
import pytest

import workloads as wl
from _parity import BF16_TOL_LSE, BF16_TOL_O, run
from test_gpu_parity import SMALL_BF16, _ok_bf16

pytestmark = pytest.mark.gpu

JOINT_SMALL = [
    # (geometry, chunk, switches): the S scale frames; scale and window
    # frames together; three ragged streams; no window (W = 0); head and
    # tail special ranges
    (1, 3, {}),
    (1, 6, {}),
    (2, 3, {}),
    (5, 2, {}),
    (4, 2, {}),
    (0, 4, {"cross_frame_special": False}),
]


@pytest.mark.parametrize("i", range(len(JOINT_SMALL)))
def test_joint_small_every_frame(gpu, i):
    g, n, sw = JOINT_SMALL[i]
    w = wl.Workload(f"joint{i}", layers=2, head_dim=64, dtype="bf16", seed=80 + i,
                    **SMALL_BF16[g], **sw)
    worst = run(w, first_chunk=n, pools_at=[n - 1, w.frames - 1],
                cache_kw={"max_frames_per_step": n}, dense_at={n - 1})
    _ok_bf16(worst)
    assert worst.cross_o <= BF16_TOL_O and worst.cross_lse <= BF16_TOL_LSE


def test_joint_main_224(gpu):
    """The 8 scale frames of the 224x224 workload jointly (2096 query rows
    over 2096 keys), then 312 single frames; every row of the chunk step
    against the dense float32 path as well."""
    w = wl.MAIN
    n = w.scale_frames
    worst = run(w, first_chunk=n, attend=lambda t: t in {7, 8, 71, 72, 319},
                heads_checked=[0, 9], pools_at=[7, 319], dense_at={7},
                cache_kw={"max_frames_per_step": n})
    _ok_bf16(worst)
    assert worst.cross_o <= BF16_TOL_O and worst.cross_lse <= BF16_TOL_LSE


def test_joint_large_518x378(gpu):
    """Four streams of 999 + 6 tokens, 8 frames jointly (8040 query rows per
    stream), then two single frames."""
    w = wl.LARGE.replace(frames=10)
    n = w.scale_frames
    worst = run(w, first_chunk=n, heads_checked=[4], pools_at=[9],
                cache_kw={"max_frames_per_step": n})
    _ok_bf16(worst)


def test_joint_per_stream_append(gpu):
    """Each stream's chunk written with its own append_frame call ([n*T]
    rows), the plan then reaching the device with the attention call."""
    w = wl.Workload("joint_ps", layers=2, head_dim=64, dtype="bf16", seed=95,
                    **SMALL_BF16[2])
    _ok_bf16(run(w, first_chunk=3, per_stream_append=True, pools_at=[2, w.frames - 1],
                 cache_kw={"max_frames_per_step": 3}))
