// Device-side lookup of a visible token through the page table.
//
// The visible tokens of a stream are, in order, every listed patch page
// whole (P tokens each), then the visible special tokens ([p1] "How the Paged
// KV Cache Attention Mechanism Enables Long Sequence Inference in
// LingBot-Map", §Building the Visible Page Table): the head (from slot 0 of
// the first listed special page) and the tail (from its first slot in the
// page after the head's pages).  Token j maps to a page of the patch or the
// special pool and a slot in it; the K row of that slot starts at
// ((page * 2 + 0) * page_size + slot) * H * D elements and the V row
// page_size * H * D elements later (pool layout [pages][2][size][H][D]).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.h"

namespace psw {

// q = j / d for 0 <= j < 2^24 and 1 <= d: float reciprocal, then one
// correction step each way (the float quotient is off by at most one).
__device__ __forceinline__ int div_small(int j, int d, float inv_d) {
  int q = static_cast<int>(static_cast<float>(j) * inv_d);
  int r = j - q * d;
  if (r < 0) { --q; r += d; }
  if (r >= d) { ++q; }
  return q;
}

// Page id of entry pi of a stream's special head (tail = false) or tail
// (tail = true): consecutive ids from a base in the compact form, else from
// the list (the tail's entries follow the head's kWSpecialHeadPages).
__device__ __forceinline__ int special_page(const AttnArgs& a, const int32_t* w, bool tail,
                                            int pi) {
  if (a.special_compact != 0) return (tail ? w[kWSpecialTailBase] : w[kWSpecialOff]) + pi;
  return a.special_ids[w[kWSpecialOff] + (tail ? w[kWSpecialHeadPages] : 0) + pi];
}

// Element offsets of token j's K and V rows (head 0) in its pool; sets
// *special when it lives in the special pool.
__device__ __forceinline__ void token_offsets(const AttnArgs& a, const int32_t* w,
                                              int j, int64_t* k_off, int64_t* v_off,
                                              bool* special) {
  const int64_t HD = static_cast<int64_t>(a.heads) * a.head_dim;
  const int patch_tok = w[kWPatchTok];
  if (j < patch_tok) {
    const int pi = div_small(j, a.patch_page, a.inv_patch_page);
    const int slot = j - pi * a.patch_page;
    const int64_t page = a.patch_ids[w[kWPatchOff] + pi];
    *k_off = (page * 2 * a.patch_page + slot) * HD;
    *v_off = *k_off + static_cast<int64_t>(a.patch_page) * HD;
    *special = false;
  } else {
    const int s = j - patch_tok;   // index among the visible special tokens
    const int head = w[kWSpecialHead];
    const bool tail = s >= head;
    const int u = tail ? s - head + w[kWSpecialTailFirst] : s;
    const int pi = div_small(u, a.special_page, a.inv_special_page);
    const int slot = u - pi * a.special_page;
    const int64_t page = special_page(a, w, tail, pi);
    *k_off = (page * 2 * a.special_page + slot) * HD;
    *v_off = *k_off + static_cast<int64_t>(a.special_page) * HD;
    *special = true;
  }
}

}  // namespace psw
