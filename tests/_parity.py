"""Drives the HIP library and the oracle through the same workload, step by
step, and compares them (used by the GPU parity tests).

Both sides receive the same seeded inputs from ``workloads``.  Page tables,
free lists, stats and pool bytes must match exactly; attention outputs within
the stated tolerances.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Callable, Iterable, Optional, Sequence

import numpy as np

import workloads as wl
from oracle.attention import gather_visible_kv, paged_attention
from oracle.cache import OracleCache

# Tolerances: bf16 inputs with float accumulation (max-abs on o and lse),
# plus a relative Frobenius bound that still bites when |o| is small.
BF16_TOL_O = 1e-2
BF16_TOL_LSE = 1e-3
BF16_TOL_REL = 2e-2
FP32_TOL = 1e-4


@dataclasses.dataclass
class Worst:
    o: float = 0.0
    lse: float = 0.0
    rel: float = 0.0
    scaled: float = 0.0     # max |o - o_ref| / (|o_ref| + max |v|)
    checked: int = 0
    # dense float32 check path: its o/lse against the float64 oracle, and
    # the paged kernel's o/lse against it (every row and head)
    dense_o: float = 0.0
    dense_lse: float = 0.0
    cross_o: float = 0.0
    cross_lse: float = 0.0
    dense_checked: int = 0
    fused_steps: int = 0    # layer steps run as one append + attention launch
    # token-exact check (identical keys, one-hot coded values): lse against
    # s + ln(Lkv), o * Lkv against the class counts, o against counts / Lkv
    # in units of its rounding bound
    exact_lse: float = 0.0
    exact_count: float = 0.0
    exact_o: float = 0.0
    exact_checked: int = 0

    def update(self, o, o_ref, lse, lse_ref, vmax=None):
        self.o = max(self.o, float(np.abs(o - o_ref).max()))
        if vmax is not None:
            self.scaled = max(self.scaled, float(
                (np.abs(o - o_ref) / (np.abs(o_ref) + vmax)).max()))
        self.lse = max(self.lse, float(np.abs(lse - lse_ref).max()))
        den = float(np.linalg.norm(o_ref.astype(np.float64)))
        num = float(np.linalg.norm((o - o_ref).astype(np.float64)))
        self.rel = max(self.rel, num / max(den, 1e-30))
        self.checked += 1


def _tables_equal(tg: dict, to) -> None:
    for key in ("qo_indptr", "patch_indptr", "patch_ids", "special_indptr",
                "special_ids", "special_last_len", "special_head_len",
                "special_tail_first", "special_tail_len"):
        assert np.array_equal(tg[key], getattr(to, key)), key


def to_np(x) -> np.ndarray:
    import torch
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return wl.bf16_bits_to_f32(x.view(torch.int16).numpy().view(np.uint16))
    return x.numpy()


def pool_bytes(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run(w: wl.Workload, *, n_frames: Optional[int] = None,
        attend: Callable[[int], bool] = lambda t: True,
        layers_checked: Optional[Sequence[int]] = None,
        heads_checked: Optional[Sequence[int]] = None,
        keyframes: Optional[Sequence[np.ndarray]] = None,
        q_scale: float = 1.0, pools_at: Iterable[int] = (),
        table_hook=None, cache_kw=None, log_every: int = 0,
        per_stream_append: bool = False, dense_at: Iterable[int] = (),
        first_chunk: int = 1, fused: bool = False, exact: bool = False,
        on_plan=None) -> Worst:
    """Streams ``w`` through both sides; returns the worst differences.

    ``per_stream_append``: write each stream's frame with its own
    append_frame call (the plan then reaches the device with the attention
    call) instead of one append_frames call for the batch.
    ``dense_at``: frames where the dense float32 check path also runs (on
    the checked layers): its gathered K/V must equal the oracle's gather bit
    for bit, and its o/lse are compared with the float64 oracle and with the
    paged kernel's output.
    ``first_chunk``: frames 0 .. first_chunk-1 are begun, written and
    attended as one joint-prefill chunk (T rows per frame), the rest one by
    one; ``attend`` and the frame sets name a step by its last frame.
    ``fused``: append and attention through psw_append_attention (one launch
    when the plan fits; ``Worst.fused_steps`` counts those).
    ``exact``: inputs from ``workloads.frame_qkv_coded`` (every key of a head
    the same vector, every value row one-hot by the token's class) and, on the
    attended frames, the closed form of that case instead of the oracle's
    attention: all weights are equal, so lse = s + ln(Lkv) and
    o[h, d] = (visible tokens of class 64h + d) / Lkv, with the visible tokens
    taken from the oracle's table and pools (see ``_exact_check``).
    ``on_plan(t, cache)``: called after each step's plan (to record it)."""
    import torch
    from paged_sliding_window_append_amd import Cache

    dev = "cuda:0"
    n = n_frames or w.frames
    layers_checked = list(range(w.layers)) if layers_checked is None \
        else list(layers_checked)
    heads = list(range(w.heads)) if heads_checked is None else list(heads_checked)
    pools_at = set(pools_at)
    dense_at = set(dense_at)
    gc = Cache.for_workload(w, device=dev, **(cache_kw or {}))
    oc = OracleCache.for_workload(w.replace(layers=1))
    # the oracle only keeps the layers it checks
    oc.patch_pool = {l: oc.patch_pool[0] if i == 0 else
                     np.zeros_like(oc.patch_pool[0])
                     for i, l in enumerate(layers_checked)}
    oc.special_pool = {l: oc.special_pool[0] if i == 0 else
                       np.zeros_like(oc.special_pool[0])
                       for i, l in enumerate(layers_checked)}
    worst = Worst()
    steps = [list(range(first_chunk))] + [[t] for t in range(first_chunk, n)]
    assert keyframes is None or first_chunk == 1
    for frames in steps:
        t = frames[-1]
        for b in range(w.streams):
            if keyframes is not None:
                gc.set_defer_eviction(b, True)
                oc.set_defer(b, True)
            if len(frames) > 1:
                gc.begin_frames(b, len(frames))
                oc.begin_frames(b, len(frames))
            else:
                gc.begin_frame(b)
                oc.begin_frame(b)
            gc.evict_frames(b)
            oc.evict(b)
        tg = gc.build_visible_page_table()
        to = oc.build_table()
        _tables_equal(tg, to)
        if table_hook is not None:
            tg = table_hook(t, tg)
            gc.set_page_table(tg)
            to = type(to)(**{k: np.asarray(v, np.int32) for k, v in tg.items()})
        gc.plan()
        if on_plan is not None:
            on_plan(t, gc)
        active = [b for b in range(w.streams)
                  if tg["qo_indptr"][b + 1] > tg["qo_indptr"][b]]
        for layer in range(w.layers):
            checked = layer in layers_checked
            if checked:
                gen = (lambda b, f: wl.frame_qkv_coded(w, b, f, layer)) if exact else \
                    (lambda b, f: wl.frame_qkv_tensors(w, b, f, layer, q_scale))
                qkv = [tuple(torch.cat(x) for x in zip(*(gen(b, f) for f in frames)))
                       for b in active]
            else:   # layers nobody compares: any data of the right shape
                shape = (len(frames) * w.tokens_per_frame, w.heads, w.head_dim)
                tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
                qkv = [tuple(torch.randn(shape, device=dev).to(tdt)
                             for _ in range(3)) for b in active]
            q = torch.cat([x[0] for x in qkv]).to(dev) if qkv else None
            k = torch.cat([x[1] for x in qkv]).to(dev) if qkv else None
            v = torch.cat([x[2] for x in qkv]).to(dev) if qkv else None
            if qkv and fused:
                pass   # append and attention in one call below
            elif qkv and per_stream_append:
                for i, b in enumerate(active):
                    gc.append_frame(layer, b, qkv[i][1].to(dev), qkv[i][2].to(dev))
            elif qkv:
                gc.append_frames(layer, k, v)
            if checked:
                for i, b in enumerate(active):
                    oc.append_frame(layer, b, wl.as_numpy(qkv[i][1]),
                                    wl.as_numpy(qkv[i][2]))
            if not qkv:
                continue
            if fused:
                worst.fused_steps += int(gc.plan_fused())
                o, lse = gc.append_attention(layer, k, v, q)
            else:
                o, lse = gc.attention(layer, q)
            if checked and attend(t) and exact:
                torch.cuda.synchronize()
                _exact_check(oc, to, layer, wl.as_numpy(q.cpu()), o, lse, active,
                             worst, 1.0 / np.sqrt(w.head_dim))
            elif checked and attend(t):
                qn = wl.as_numpy(q.cpu())[:, heads]
                pp = oc.patch_pool[layer][:, :, :, heads]
                sp = oc.special_pool[layer][:, :, :, heads]
                o_ref, lse_ref = paged_attention(pp, sp, to, qn)
                vmax = max(float(np.abs(wl.bf16_bits_to_f32(x[:, 1]) if
                                        x.dtype == np.uint16 else x[:, 1]).max())
                           for x in (pp, sp))
                torch.cuda.synchronize()
                worst.update(to_np(o)[:, heads], o_ref,
                             to_np(lse)[:, heads], lse_ref, vmax)
            if checked and t in dense_at:
                _dense_check(gc, oc, to, layer, q, o, lse, heads, active, worst)
            if checked and t in pools_at:
                assert np.array_equal(pool_bytes(gc.patch_pools[layer]),
                                      oc.patch_pool[layer]), "patch pool"
                assert np.array_equal(pool_bytes(gc.special_pools[layer]),
                                      oc.special_pool[layer]), "special pool"
        if keyframes is not None:
            for b in range(w.streams):
                if keyframes[b][t]:
                    gc.execute_deferred_eviction(b)
                    oc.execute_deferred_eviction(b)
                else:
                    gc.rollback_last_frame(b)
                    oc.rollback_last_frame(b)
                gc.set_defer_eviction(b, False)
                oc.set_defer(b, False)
        for b in range(w.streams):
            assert gc.stats(b) == oc.stats(b)
            assert gc.free_list(b) == oc.free_list(b)
        if log_every and (t % log_every == 0 or t == n - 1):
            print(f"  frame {t}: worst o {worst.o:.3g} lse {worst.lse:.3g} "
                  f"rel {worst.rel:.3g} ({worst.checked} checks)", flush=True)
            sys.stdout.flush()
    torch.cuda.synchronize()
    gc.close()
    return worst


BF16_ONE = 0x3F80   # bfloat16 bits of 1.0


def _exact_check(oc, to, layer, q, o, lse, active, worst, sm_scale) -> None:
    """Closed form of attention when every key of a head is the same vector
    (so every weight is 1 / Lkv) and every value row is one-hot.

    For each active stream the oracle's gather gives the visible K and V
    rows.  The check first confirms the premise on them (all K rows equal,
    every V row a single 1.0), then compares with the GPU result:
      lse[i, h] = q[i, h] . key[h] * sm_scale + ln(Lkv), within 1e-5 (one
        token more or less moves it by 1 / Lkv: 4.9e-5 at 20 352 tokens);
      o[i, h, d] * Lkv = n[h, d], the visible tokens of class 64h + d: the
        largest |o * Lkv - n| must stay below 0.5, so every count is
        recovered exactly (counts stay far below 2^8, where one bf16
        rounding of o moves o * Lkv by less than 0.5), and a token dropped,
        added or read from another token's place changes a count by 1;
      |o - n / Lkv| within one bf16 rounding of the output (2^-9 relative)
        plus the fp16 rounding of split partials (2^-12 of the row's largest
        value), doubled: reported as a ratio that must be <= 1."""
    o_np, lse_np = to_np(o), to_np(lse)
    for b in active:
        r0, r1 = int(to.qo_indptr[b]), int(to.qo_indptr[b + 1])
        kk, vv = gather_visible_kv(oc.patch_pool[layer], oc.special_pool[layer], to, b)
        L, H, D = kk.shape
        assert L > 0
        k64 = kk.reshape(L, -1).view(np.uint64)
        assert (k64 == k64[:1]).all(), "keys not identical"
        nz = np.flatnonzero(vv)        # one element per row, of value 1.0
        assert nz.size == L and (vv.reshape(-1)[nz] == BF16_ONE).all() and \
            np.array_equal(nz // (H * D), np.arange(L)), "values not one-hot"
        counts = np.bincount(nz % (H * D), minlength=H * D).reshape(H, D).astype(np.float64)
        key = wl.bf16_bits_to_f32(kk[0]).astype(np.float64)       # [H, D]
        qb = wl.bf16_bits_to_f32(q[r0:r1]).astype(np.float64)     # [rows, H, D]
        s = np.einsum("rhd,hd->rh", qb, key) * sm_scale
        lse_exp = s + np.log(L)
        ob = o_np[r0:r1].astype(np.float64)
        o_exp = counts / L
        worst.exact_lse = max(worst.exact_lse, float(np.abs(lse_np[r0:r1] - lse_exp).max()))
        worst.exact_count = max(worst.exact_count, float(np.abs(ob * L - counts).max()))
        bound = 2.0 * (2.0 ** -9 * o_exp + 2.0 ** -12 * o_exp.max(axis=1, keepdims=True))
        # a head with no token of any of its classes has bound 0 and must
        # give exactly 0 there (inf otherwise, never NaN, which max() skips)
        err = np.abs(ob - o_exp)
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
        worst.exact_o = max(worst.exact_o, float(ratio.max()))
    worst.exact_checked += 1


def _dense_check(gc, oc, to, layer, q, o, lse, heads, active, worst) -> None:
    import torch
    kd, vd = gc.gather_visible_f32(layer)
    kvp = gc.visible_tokens()
    kd_np, vd_np = kd.cpu().numpy(), vd.cpu().numpy()
    for b in range(len(kvp) - 1):
        r0, r1 = int(kvp[b]), int(kvp[b + 1])
        if b not in active:
            assert r1 == r0, "inactive stream with visible tokens"
            continue
        kref, vref = gather_visible_kv(oc.patch_pool[layer], oc.special_pool[layer],
                                       to, b)
        widen = wl.bf16_bits_to_f32 if kref.dtype == np.uint16 else \
            (lambda x: x.astype(np.float32))
        assert r1 - r0 == kref.shape[0], "visible token count"
        assert np.array_equal(kd_np[r0:r1], widen(kref)), "gathered K"
        assert np.array_equal(vd_np[r0:r1], widen(vref)), "gathered V"
    od, lsed = gc.dense_attention_f32(q, kd, vd)
    qn = wl.as_numpy(q.cpu())[:, heads]
    o64, lse64 = paged_attention(oc.patch_pool[layer][:, :, :, heads],
                                 oc.special_pool[layer][:, :, :, heads], to, qn,
                                 acc=np.float64)
    torch.cuda.synchronize()
    od_np, lsed_np = od.cpu().numpy(), lsed.cpu().numpy()
    worst.dense_o = max(worst.dense_o, float(np.abs(od_np[:, heads] - o64).max()))
    worst.dense_lse = max(worst.dense_lse,
                          float(np.abs(lsed_np[:, heads] - lse64).max()))
    worst.cross_o = max(worst.cross_o, float(np.abs(to_np(o) - od_np).max()))
    worst.cross_lse = max(worst.cross_lse, float(np.abs(to_np(lse) - lsed_np).max()))
    worst.dense_checked += 1
