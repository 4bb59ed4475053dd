"""The library from a plain C program on the GPU (tests/c/abi_device.c, built
by __graft_entry__.build() into _build/abi_device): device memory from the
HIP runtime's C API, every step of each frame through the C ABI, no Python
or torch in the caller.  Two streams, four heads, 12 frames that
span several 64-key tiles and split the keys (so the merge runs); each
frame's o and lse must match the oracle within the bf16 tolerances, the same
bar as the other parity tests ([p1] §FlashInfer Kernel Execution, §Building
the Visible Page Table)."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import workloads as wl
from oracle.attention import paged_attention
from oracle.cache import OracleCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "_build", "abi_device")
MAGIC = 0x70737731

W = wl.Workload("c_abi", layers=1, heads=4, head_dim=64, dtype=wl.BF16,
                tokens_per_frame=70, num_special=6, special_page=8, scale_frames=2,
                sliding_window=5, frames=12, streams=2)


@pytest.mark.gpu
def test_c_caller_on_the_gpu_matches_oracle(gpu, tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("_build/abi_device is not built: run __graft_entry__.build()")
    w = W
    rows, H, D = w.streams * w.tokens_per_frame, w.heads, w.head_dim
    inputs = []
    with open(tmp_path / "in.bin", "wb") as f:
        np.array([MAGIC, w.frames, w.streams, w.tokens_per_frame, w.num_special,
                  w.special_page, w.scale_frames, w.sliding_window, H, D, w.pmax, w.smax],
                 dtype=np.int32).tofile(f)
        for t in range(w.frames):
            per = [wl.frame_qkv(w, b, t, 0) for b in range(w.streams)]
            qkv = [np.concatenate([p[i] for p in per]) for i in range(3)]
            inputs.append(qkv)
            for x in qkv:
                np.ascontiguousarray(x, dtype=np.uint16).tofile(f)
    print("running _build/abi_device on", w, flush=True)
    r = subprocess.run([EXE, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint8)
    o_bytes, l_bytes = rows * H * D * 2, rows * H * 4
    assert out.size == w.frames * (o_bytes + l_bytes)

    oc = OracleCache.for_workload(w)
    worst_o = worst_l = 0.0
    for t in range(w.frames):
        for b in range(w.streams):
            oc.begin_frame(b)
            oc.evict(b)
        table = oc.build_table()
        q, k, v = inputs[t]
        for b in range(w.streams):
            sl = slice(b * w.tokens_per_frame, (b + 1) * w.tokens_per_frame)
            oc.append_frame(0, b, k[sl], v[sl])
        o_ref, lse_ref = paged_attention(oc.patch_pool[0], oc.special_pool[0], table, q)
        rec = out[t * (o_bytes + l_bytes):(t + 1) * (o_bytes + l_bytes)]
        o = wl.bf16_bits_to_f32(rec[:o_bytes].view(np.uint16)).reshape(rows, H, D)
        lse = rec[o_bytes:].view(np.float32).reshape(rows, H)
        worst_o = max(worst_o, float(np.abs(o - o_ref).max()))
        worst_l = max(worst_l, float(np.abs(lse - lse_ref).max()))
    print(f"worst o {worst_o:.3g} lse {worst_l:.3g}", flush=True)
    assert worst_o <= 1e-2
    assert worst_l <= 1e-3
