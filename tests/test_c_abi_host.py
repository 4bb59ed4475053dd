"""The C ABI from plain C (no Python in the caller, no device): tests/c/
abi_host.c is built with gcc against include/psw.h and libpsw.so, drives two
streams through frame allocation, eviction, deferred eviction with commit or
rollback and the visible page table, and prints every table, stats record and
free list.  Each must equal the oracle's for the same call sequence ([p1]
§Building the Visible Page Table; [p3] §Monitoring Cache Statistics; [p4]
§Deferred Eviction and Rollback Mechanism); the error paths return the
documented codes."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from oracle.cache import OracleCache
from paged_sliding_window_append_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PSW_EINVAL, PSW_ESTATE = -1, -4


@pytest.fixture(scope="module")
def abi_host(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpsw.so is not built")
    exe = str(tmp_path_factory.mktemp("abi") / "abi_host")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O1",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"),
                    "-L", lib_dir, "-lpsw", f"-Wl,-rpath,{lib_dir}", "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def oracle_records(cross: bool, frames: int):
    """The oracle's records for the call sequence of abi_host.c."""
    oc = OracleCache(layers=1, streams=2, heads=2, head_dim=64, tokens_per_frame=22,
                     num_special=6, special_page=8, scale_frames=2, sliding_window=4,
                     pmax=8, smax=32, include_scale_frames=True,
                     cross_frame_special=cross)
    out = []
    for t in range(frames):
        deferred = t % 3 == 2
        for b in range(2):
            if b == 1 and deferred:
                oc.set_defer(b, True)
            oc.begin_frame(b)
            oc.evict(b)
        tb = oc.build_table()
        for b in range(2):
            ps = tb.patch_ids[tb.patch_indptr[b]:tb.patch_indptr[b + 1]]
            ss = tb.special_ids[tb.special_indptr[b]:tb.special_indptr[b + 1]]
            out.append(" ".join(
                ["T", str(t), str(b), str(tb.qo_indptr[b]), str(tb.qo_indptr[b + 1]), "|"] +
                [str(x) for x in ps] + ["|"] + [str(x) for x in ss] + ["|"] +
                [str(tb.special_last_len[b]), str(tb.special_head_len[b]),
                 str(tb.special_tail_first[b]), str(tb.special_tail_len[b])]))
        if deferred:
            if t % 6 == 2:
                oc.execute_deferred_eviction(1)
            else:
                oc.rollback_last_frame(1)
            oc.set_defer(1, False)
        for b in range(2):
            st = oc.stats(b)
            out.append(" ".join(["S", str(t), str(b)] + [str(st[k]) for k in (
                "frame_count", "scale_pages", "live_pages", "free_pages", "special_tokens")]))
            out.append(" ".join(["L", str(t), str(b)] + [str(x) for x in oc.free_list(b)]))
    return out


@pytest.mark.parametrize("cross", [True, False])
def test_c_caller_matches_oracle(abi_host, cross):
    frames = 40
    r = subprocess.run([abi_host, str(int(cross)), str(frames)], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = [" ".join(x.split()) for x in r.stdout.splitlines()]
    recs = [x for x in lines if not x.startswith("E ")]
    want = oracle_records(cross, frames)
    assert len(recs) == len(want)
    for got, exp in zip(recs, want):
        assert got == exp
    errors = dict(x.split()[1:] for x in lines if x.startswith("E "))
    assert errors == {"rollback_after_eviction": str(PSW_ESTATE),
                      "rollback_twice": str(PSW_ESTATE),
                      "bad_stream": str(PSW_EINVAL),
                      "plan_without_table": str(PSW_ESTATE)}
