"""CPU checks of the token-exact closed form used by the GPU tests
(``_parity._exact_check``): the oracle's own attention on the coded inputs
passes it, and one token dropped or read from the wrong page -- planted in
the oracle's table, on the CPU -- fails it."""
import numpy as np
import pytest
import torch

import workloads as wl
from _parity import Worst, _exact_check
from oracle.attention import paged_attention
from oracle.cache import OracleCache

W = wl.Workload("coded", layers=1, heads=2, head_dim=64, dtype="bf16",
                tokens_per_frame=70, num_special=6, special_page=16,
                scale_frames=2, sliding_window=5, frames=12, streams=2, seed=5)


def _stream(upto):
    oc = OracleCache.for_workload(W)
    for t in range(upto + 1):
        for b in range(W.streams):
            oc.begin_frame(b)
            oc.evict(b)
        to = oc.build_table()
        qs = []
        for b in range(W.streams):
            q, k, v = wl.frame_qkv_coded(W, b, t, 0)
            oc.append_frame(0, b, wl.as_numpy(k), wl.as_numpy(v))
            qs.append(wl.as_numpy(q))
    return oc, to, np.concatenate(qs)


def _oracle_result(oc, to, q):
    o, lse = paged_attention(oc.patch_pool[0], oc.special_pool[0], to, q)
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse)


def _check(oc, to, q, o, lse):
    worst = Worst()
    _exact_check(oc, to, 0, q, o, lse, range(W.streams), worst,
                 1.0 / np.sqrt(W.head_dim))
    return worst


def test_coded_inputs_premise():
    q, k, v = wl.frame_qkv_coded(W, 0, 3, 0)
    assert torch.equal(k, k[:1].expand_as(k))
    vf = v.float().reshape(W.tokens_per_frame, -1)
    assert torch.equal(vf.sum(dim=1), torch.ones(W.tokens_per_frame))
    assert set(vf.unique().tolist()) == {0.0, 1.0}


@pytest.mark.parametrize("t", [0, 4, 11])
def test_oracle_satisfies_closed_form(t):
    oc, to, q = _stream(t)
    o, lse = _oracle_result(oc, to, q)
    worst = _check(oc, to, q, o, lse)
    assert worst.exact_checked == 1
    assert worst.exact_lse <= 1e-5
    assert worst.exact_count < 0.5
    assert worst.exact_o <= 1.0


def test_dropped_token_is_caught():
    """The result of a table missing the last visible special token."""
    oc, to, q = _stream(11)
    bad = type(to)(**{k: np.array(v, copy=True) for k, v in vars(to).items()})
    assert bad.special_tail_len[0] == 0 and bad.special_last_len[0] > 1
    bad.special_head_len[0] -= 1
    bad.special_last_len[0] -= 1
    o, lse = _oracle_result(oc, bad, q)
    worst = _check(oc, to, q, o, lse)
    assert worst.exact_lse > 1e-5
    assert worst.exact_count >= 0.5


def test_wrong_page_is_caught():
    """The result of a table whose first window page is replaced by a free
    (stale) page of the same stream."""
    oc, to, q = _stream(11)
    bad = type(to)(**{k: np.array(v, copy=True) for k, v in vars(to).items()})
    free = oc.free_list(0)
    assert free
    bad.patch_ids[W.scale_frames] = free[-1]
    o, lse = _oracle_result(oc, bad, q)
    worst = _check(oc, to, q, o, lse)
    assert worst.exact_count >= 0.5
