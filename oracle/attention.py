"""Attention of one frame's queries over the visible pages (oracle, tests only).

The attention runs only over the pages listed in the visible page table, so
its work follows the window, not the video length ([p1] §FlashInfer Kernel
Execution; [p3] §Visible Page Table Attention and §Custom CUDA Kernel
Implementation).  The pages also describe a validation mode that gathers the
paged K/V into dense tensors and runs ordinary attention in float32
([p1] §Memory Efficiency Analysis, "Precision modes"); this oracle is that
mode written out: gather through the table, then plain softmax attention.

Readings (the pages state none of these): scale 1/sqrt(D); no mask inside the
visible set (the frame's own tokens are visible to all its queries, the past
only through the cache); one KV head per query head; the log-sum-exp is the
natural logarithm of the softmax denominator of the scaled scores.
"""
from __future__ import annotations

import numpy as np


def _widen(x: np.ndarray, acc) -> np.ndarray:
    """Stored elements -> accumulation dtype.  uint16 holds bfloat16 bits."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(acc, copy=False)


def gather_visible_kv(patch_pool: np.ndarray, special_pool: np.ndarray,
                      table, b: int):
    """K and V ([Lkv, H, D], stored dtype) of stream b, in table order:
    every listed patch page whole, then the visible special tokens -- the
    head range from slot 0 of the first listed special page, then the tail
    range from its first slot in the page after the head's pages."""
    p0, p1 = table.patch_indptr[b], table.patch_indptr[b + 1]
    s0, s1 = table.special_indptr[b], table.special_indptr[b + 1]
    ks, vs = [], []
    for pid in table.patch_ids[p0:p1]:
        ks.append(patch_pool[pid, 0])
        vs.append(patch_pool[pid, 1])
    Ps = special_pool.shape[2]
    sids = table.special_ids[s0:s1]
    head = int(table.special_head_len[b])
    first = int(table.special_tail_first[b])
    tail = int(table.special_tail_len[b])
    n_head_pages = -(-head // Ps)
    for part, (lo, n) in ((sids[:n_head_pages], (0, head)),
                          (sids[n_head_pages:], (first, tail))):
        if n == 0:
            continue
        kk = np.concatenate([special_pool[sid, 0] for sid in part], axis=0)
        vv = np.concatenate([special_pool[sid, 1] for sid in part], axis=0)
        ks.append(kk[lo:lo + n])
        vs.append(vv[lo:lo + n])
    H, D = patch_pool.shape[3], patch_pool.shape[4]
    if not ks:
        empty = np.zeros((0, H, D), dtype=patch_pool.dtype)
        return empty, empty.copy()
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      sm_scale: float, acc=np.float32):
    """Plain attention of q [Tq, D] over k, v [Lkv, D] in ``acc`` precision.

    Two passes over the scores: the row maximum, then the exponentials, their
    sum and the weighted sum of values.  Returns (o [Tq, D], lse [Tq])."""
    s = (q @ k.T) * acc(sm_scale)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def paged_attention(patch_pool: np.ndarray, special_pool: np.ndarray,
                    table, q: np.ndarray, sm_scale: float | None = None,
                    acc=np.float32):
    """Paged prefill attention for every stream in the table.

    q: [sum T_b, H, D] query rows, stream after stream (``qo_indptr``).
    Returns (o [sum T_b, H, D], lse [sum T_b, H]) in ``acc`` precision."""
    Tq, H, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    o = np.zeros((Tq, H, D), dtype=acc)
    lse = np.zeros((Tq, H), dtype=acc)
    B = len(table.qo_indptr) - 1
    for b in range(B):
        r0, r1 = int(table.qo_indptr[b]), int(table.qo_indptr[b + 1])
        if r1 == r0:
            continue
        k, v = gather_visible_kv(patch_pool, special_pool, table, b)
        qb, k, v = _widen(q[r0:r1], acc), _widen(k, acc), _widen(v, acc)
        for h in range(H):
            o[r0:r1, h], lse[r0:r1, h] = softmax_attention(
                qb[:, h], k[:, h], v[:, h], sm_scale, acc)
    return o, lse
