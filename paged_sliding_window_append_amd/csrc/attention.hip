// bf16 paged prefill attention for gfx950 (CDNA4), head_dim 64.
//
// What it computes ([p1] "How the Paged KV Cache Attention Mechanism
// Enables Long Sequence Inference in LingBot-Map", §FlashInfer Kernel
// Execution; [p3] "FlashInfer Paged KV Cache Performance Benefits in
// LingBot-Map", §Visible Page Table Attention): every query row of the
// current frame attends to the visible tokens listed in the page table --
// scale pages, window pages, then the special pages -- reading K/V straight
// from the pages, with no dense gather.
//
// Work split.  A workgroup (4 waves) takes one work item (stream, block of
// up to 272 query rows, range of visible tokens) for one head.  Rows come in
// 16-row tiles: wave w owns tiles w, w+4, w+8, w+12 for every key; a 17th
// tile (rows 256..271) is shared, each wave taking one 16-key quarter of
// every key tile, and the four partial results are merged at the end.
//
// Key tiles of 64 tokens go global -> LDS with 16-byte direct loads (no
// register staging), double-buffered, one barrier per tile.  Each LDS row
// holds one token (64 bf16 = 128 B) with its eight 16-byte chunks permuted by
// swz(row): row bits 4, 1, 3 flip chunk bits 0, 1, 2.  With 64 four-byte
// banks the 16 lanes of one lane group then read 16 distinct bank groups for
// a K fragment, and the 32 lanes of one transposed V read are conflict-free.
// The K reads still measure 4 conflict cycles each (SQ_LDS_BANK_CONFLICT): a
// 16-byte read is served in 8-byte halves, 32 lanes at a time, so lane groups
// 0 and 1 both use banks 0-1 (mod 4) in the first half.  Reading K as two
// 8-byte halves, odd lane groups the second one first (and their Q fragments
// swapped to match), removes the conflicts but issues twice the LDS
// instructions, and the kernel measured 5% slower that way.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16; lane l, g = l/16, r = l%16): the
// A operand row r holds k-slots 8g..8g+7, the B operand column r the same
// k-slots, and accumulator element i of lane l is row 4g+i, column r.
//  * Scores are computed transposed, S^T = K Q^T, so a lane holds 8 keys of
//    one query per 32-key half and the row max needs two cross-lane steps.
//    The K row fed to A row r of key block kb is
//      32*(kb/2) + 8*(r/4) + 4*(kb%2) + r%4,
//    which leaves lane group g holding keys 32c + 8g + 0..7 of half c:
//    exactly the k-slots the B operand of O^T += V^T P^T wants, so P stays
//    in its lanes.
//  * V^T comes from row-major V in LDS through ds_read_b64_tr_b16: within a
//    16-lane group, lane i receives element i%4 of the 8-byte chunks read by
//    lanes 4j + i/4 (j = 0..3), which turns four 4-wide row pieces into the
//    column the A operand needs.
//  * The row sums add the float weights before their bf16 rounding: a
//    rounded sum could move the log-sum-exp by up to 2^-9.
//
// Softmax: scores stay raw; p = 2^(s*c - m*c) with c = sm_scale*log2(e) and
// m a running reference, not necessarily the exact running max.  The
// weights of each lane's 8 keys are computed against the current m and
// summed (the sum is needed anyway); as long as that sum stays at or below
// 2^kSumLog2 no weight overflowed, and nothing else is done.  Otherwise (a
// score far above m) the half is redone: exact row max, m moved to it,
// accumulators rescaled, weights recomputed.  In the first tile, where m is
// still the sentinel, the row max is taken before the weights instead.  So
// the row max costs nothing in the common case and the weights stay below
// 2^kSumLog2.  m starts at a finite sentinel so no NaN can arise from
// -inf - -inf with masked keys.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "device.h"
#include "launch.h"
#include "paging.h"

namespace psw {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSumLimit = 256.0f;     // 2^kSumLog2, kSumLog2 = 8
// Fast form: with the reference fixed, a lane's running weight sum may grow
// to this before the workgroup starts over; 2^64 and the products with V stay
// far inside float and bf16 range, so nothing overflows and the relative
// precision is unchanged.
constexpr float kFixedLimit = 18446744073709551616.0f;   // 2^64
constexpr float kNoMax = -1.0e30f;       // running max before any key
// Group table entries: the K row of the group's first token (29 bits) and
// flags: rows of a frame being appended (in k/v), rows of the special pool,
// or a group whose rows are looked up one by one.
constexpr uint32_t kEntSlow = 1u << 31;
constexpr uint32_t kEntCur = 1u << 30;
constexpr uint32_t kEntSpecial = 1u << 29;
constexpr uint32_t kEntRowMask = kEntSpecial - 1;
static_assert(kMaxPoolRows == int64_t{kEntSpecial}, "29-bit rows");
constexpr int kRowBytes = 128;                 // one token's head slice
constexpr int kTileBytes = kKvTile * kRowBytes;  // 8 KiB

__device__ __forceinline__ int swz(int row) {
  return ((row >> 4) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}

// Byte offset in a tile of the 16-byte chunk `chunk` of token row `row`.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ bf16x8 lds_read16(const unsigned char* base, int off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
}

__device__ __forceinline__ i16x4 lds_read_tr(const unsigned char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max8(f32x4 a, f32x4 b) {
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
               fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
}

// Max over the four lanes l, l^16, l^32, l^48 (one query's 32 keys), two
// butterfly exchanges.
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats to a bf16 pair (round to nearest even), one instruction.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(lo);
  r[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Two floats to an fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 r;
  r[0] = static_cast<_Float16>(lo);
  r[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}



// The kernel body.  FUSED: the launch also writes the frames' K/V into the
// pools (a few 4 KiB chunks per workgroup, loaded first and stored after the
// first barrier) and reads those frames' rows from k/v instead; `f` holds the
// plan and the cuts (null otherwise).  COMPACT: the plan gives each stream's
// special pages as two runs of consecutive ids (AttnArgs::special_compact)
// instead of listing them.
template <bool FUSED, int W, bool COMPACT>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const FusedArgs* f) {
  // W waves; wave w owns query tiles w, w + W, ... (16 tiles in all), waves
  // 0..3 share the 17th
  constexpr int kWaves = W;
  constexpr int NQT = 16 / W;
  static_assert(W == 4 || W == 8, "4 or 8 waves");
  __shared__ __attribute__((aligned(16))) unsigned char kbuf0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char kbuf1[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf1[kTileBytes];

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int32_t* w = a.work + __builtin_amdgcn_workgroup_id_x() * kWorkInts;
  const int h = __builtin_amdgcn_workgroup_id_y();

  // ---- fused append: loads now, stores after the first barrier
  u32x4 cval[kFusedCopies];
  unsigned char* cdst[kFusedCopies];
  int32_t bval[4] = {0, 0, 0, 0};
  int bn = 0;   // blob ints this thread writes (workgroup 0 only)
  // chunk ci of the frames' K/V: this thread's 16 source and destination
  // bytes (false past the end of its segment)
  const int lin = __builtin_amdgcn_workgroup_id_x() +
                  __builtin_amdgcn_workgroup_id_y() * a.n_items;
  const int nwg = a.n_items * a.heads;
  auto chunk_bytes = [&](int ci, const unsigned char** src, unsigned char** dst)
      __attribute__((always_inline)) {
    const int32_t* cstart = f->data + f->off_cstart;
    const AppendSeg* segs = reinterpret_cast<const AppendSeg*>(f->data + f->off_segs);
    int sg = 0;
    while (sg + 1 < f->nseg && ci >= cstart[sg + 1]) ++sg;
    const AppendSeg seg = segs[sg];
    const int64_t off = static_cast<int64_t>(ci - cstart[sg]) * kAppendChunk + tid * 16;
    if (tid * 16 >= kAppendChunk || off >= seg.bytes) return false;
    *src = ((seg.flags & 1) ? f->v_in : f->k_in) + seg.src_off + off;
    *dst = static_cast<unsigned char*>(
               const_cast<void*>((seg.flags & 2) ? a.special_pool : a.patch_pool)) +
           seg.dst_off + off;
    return true;
  };
  // (issued after the first key tile's loads: its segment search is a chain
  // of dependent scalar loads)
  auto fused_loads = [&]() __attribute__((always_inline)) {
    if constexpr (FUSED) {
#pragma unroll
      for (int r = 0; r < kFusedCopies; ++r) {
        cdst[r] = nullptr;
        cval[r] = u32x4{0u, 0u, 0u, 0u};
        const int ci = lin + r * nwg;
        const unsigned char* src;
        if (ci < f->total_chunks && chunk_bytes(ci, &src, &cdst[r]))
          cval[r] = *reinterpret_cast<const u32x4*>(src);
      }
      if (lin == 0) {
        bn = min(4, f->blob_n - 4 * tid);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < bn) bval[i] = f->data[4 * tid + i];
      }
    }
  };
  auto fused_stores = [&]() __attribute__((always_inline)) {
    if constexpr (FUSED) {
#pragma unroll
      for (int r = 0; r < kFusedCopies; ++r)
        if (cdst[r] != nullptr) *reinterpret_cast<u32x4*>(cdst[r]) = cval[r];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < bn) f->ws_blob[4 * tid + i] = bval[i];
      // chunks beyond those held in registers (few workgroups): copied here
      for (int ci = lin + kFusedCopies * nwg; ci < f->total_chunks; ci += nwg) {
        const unsigned char* src;
        unsigned char* dst;
        if (chunk_bytes(ci, &src, &dst))
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };

  const int q_row0 = w[kWQRow0];
  const int q_rows = w[kWQRows];
  const int kv_begin = w[kWKvBegin];
  const int kv_end = w[kWKvEnd];
  const int split = w[kWSplit];
  const int patch_tok = w[kWPatchTok];
  const int32_t* patch_ids = a.patch_ids + w[kWPatchOff];
  const int32_t* special_ids = a.special_ids + w[kWSpecialOff];   // the list form
  if (q_rows <= 0 || kv_end <= kv_begin) {   // an empty (padding) item
    fused_loads();
    fused_stores();
    return;
  }

  // ---- fused: where the current frames' rows start in the visible order
  // (patch list entry, visible special index), their frame offsets, and the
  // stream's first row in k/v
  int pcut_page = 0x7fffffff, f_off_p = 0, s_cut = 0x7fffffff, f_off_s = 0, in_row0 = 0;
  if constexpr (FUSED) {
    const int b = w[kWStream];
    const int32_t* fc = f->data + f->off_fcur + 4 * b;
    pcut_page = fc[0];
    f_off_p = fc[1];
    s_cut = fc[2];
    f_off_s = fc[3];
    in_row0 = f->data[f->off_qo + b];
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int H = a.heads;
  const float c2 = a.sm_scale * kLog2e;

  const int nqt = (q_rows + kQTileRows - 1) / kQTileRows;
  const int nmain = nqt < kWaves * NQT ? nqt : kWaves * NQT;
  const bool has_tail = nqt > kWaves * NQT;
  // valid main tiles of this wave (wave-uniform)
  const int nt = nmain > wave ? (nmain - wave + kWaves - 1) / kWaves : 0;
  // Waves 4..7 of an 8-wave workgroup (no tail part, no loads) run their
  // fast tiles half a tile behind in phase (lag_tile below).
  constexpr bool kLag = kWaves == 8;
  const bool lagged = kLag && wave >= kTailWaves;

  // ---- Q^T fragments (B operand of S^T = K Q^T)
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  auto load_q = [&](int tile_row0, bf16x8* dst) {
    const int row = tile_row0 + r16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < q_rows)
        v = *reinterpret_cast<const u32x4*>(
            qg + (static_cast<int64_t>(q_row0 + row) * H + h) * 64 + kk * 32 + g * 8);
      dst[kk] = __builtin_bit_cast(bf16x8, v);
    }
  };
  bf16x8 qf[NQT][2];
  bf16x8 qt_tail[2];
  // (issued after the first tiles' page lookups, so that waiting for those
  // does not wait for these too: loads retire in issue order)
  auto load_all_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      if (t < nt) {
        load_q((wave + t * kWaves) * kQTileRows, qf[t]);
      } else {
        qf[t][0] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        qf[t][1] = qf[t][0];
      }
    }
    if (has_tail) {
      load_q(kWaves * NQT * kQTileRows, qt_tail);
    } else {
      qt_tail[0] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      qt_tail[1] = qt_tail[0];
    }
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 oacc[NQT][4];
  float l_run[NQT];   // this lane's share of the row sum (8 of 32 keys)
  float m_run[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = kNoMax;
    l_run[t] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[t][db] = zero4;
  }
  f32x4 otail[4] = {zero4, zero4, zero4, zero4};
  float ltail = 0.f;
  float mtail = kNoMax;

  // ---- global -> LDS: wave w < 4 fills token rows 16w..16w+15 of a tile, 8
  // rows per instruction; lane L writes LDS bytes [16L, 16L+16) of its 1 KiB
  // piece, i.e. chunk position L%8 of row L/8, so it fetches source chunk
  // (L%8) ^ swz(row).
  //
  // A wave's 16 rows are consecutive visible tokens.  When they lie in one
  // page (always for pages whose size is a multiple of 16 and a split start
  // that is a multiple of 64, as here), one address serves the group and
  // each lane adds a fixed offset: row * (H*D*2) + chunk * 16.  Otherwise (a
  // page boundary inside the 16 rows, the end of the range) every lane looks
  // up its own row.  The groups' sources are worked out once per workgroup,
  // all of them in parallel at the start (one 32-bit entry per group in LDS:
  // the K row of its first token in its pool, or in k/v for the rows of a
  // frame being appended, and flags), so a loading wave spends a few scalar
  // instructions per tile on its address instead of a page lookup.
  const unsigned char* pool_patch = static_cast<const unsigned char*>(a.patch_pool);
  const unsigned char* pool_special = static_cast<const unsigned char*>(a.special_pool);
  const int64_t HD = static_cast<int64_t>(H) * 64;
  const uint32_t tok_bytes = static_cast<uint32_t>(H) * 128u;   // one token, all heads
  uint32_t lane_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * wave + 8 * i + (lane >> 3);
    lane_off[i] = static_cast<uint32_t>(8 * i + (lane >> 3)) * tok_bytes +
                  static_cast<uint32_t>(((lane & 7) ^ swz(row)) << 4);
  }
  // Visible special tokens: a head from slot 0 of the first listed special
  // page, then a tail from slot sp_tail_first of list entry sp_head_pages.
  // Page ids: special_ids[entry], or in the compact form the head's or the
  // tail's base id plus the page's index in its run.
  const int sp_head = w[kWSpecialHead];
  const int sp_tail_first = w[kWSpecialTailFirst];
  const int sp_head_pages = w[kWSpecialHeadPages];
  const int ntiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;
  // entry of group q (rows 16q..16q+15) of key tile t
  auto group_entry = [&](int t, int q) -> uint32_t {
    const int j0 = kv_begin + t * kKvTile + 16 * q;
    const bool sp = j0 >= patch_tok;
    const int s0 = j0 - patch_tok;   // special index (when sp)
    const bool in_tail = sp && s0 >= sp_head;
    // position in the pool's page sequence, and the list entry it counts from
    const int jj = !sp ? j0 : in_tail ? s0 - sp_head + sp_tail_first : s0;
    const int pbase = in_tail ? sp_head_pages : 0;
    const int psize = sp ? a.special_page : a.patch_page;
    const int pi = div_small(jj, psize, sp ? a.inv_special_page : a.inv_patch_page);
    const int slot0 = jj - pi * psize;
    // one page and one range: the 16 rows may not run from the head into
    // the tail
    const bool fast = j0 + 16 <= kv_end && slot0 + 16 <= psize &&
                      (!sp || in_tail || s0 + 16 <= sp_head);
    if constexpr (FUSED) {
      if (!sp && pi >= pcut_page) {   // rows of a frame being appended: from k/v
        const int r = in_row0 + (f_off_p + pi - pcut_page) * f->tokens_per_frame +
                      f->num_special + slot0;
        return fast ? (kEntCur | static_cast<uint32_t>(r)) : kEntSlow;
      }
      if (sp && s0 + 16 > s_cut) return kEntSlow;   // may hold current rows
    }
    if (!fast) return kEntSlow;
    int page;
    if constexpr (COMPACT)   // the list is absent: never read it
      page = sp ? (in_tail ? w[kWSpecialTailBase] : w[kWSpecialOff]) + pi : patch_ids[pi];
    else
      page = sp ? special_ids[pbase + pi] : patch_ids[pi];
    const uint32_t r = static_cast<uint32_t>(page) * 2u * static_cast<uint32_t>(psize) +
                       static_cast<uint32_t>(slot0);
    return (sp ? kEntSpecial : 0u) | r;
  };
  // Filled (tiles 2 on) while the first tiles' loads are in flight, read
  // after the barrier that precedes the first tile's compute; tiles 0 and 1
  // work out their own entries.
  __shared__ uint32_t gtab[kGroupTabTiles * kLoadWaves];
  __shared__ int vote;   // some wave's fast-form sums overflowed
  auto fill_table = [&]() __attribute__((always_inline)) {
    const int nent = min(ntiles, kGroupTabTiles) * kLoadWaves;
    for (int e = 2 * kLoadWaves + tid; e < nent; e += kWaves * 64)
      gtab[e] = group_entry(e >> 2, e & 3);
  };
  // this wave's group entry of a tile (0 for waves that load nothing)
  auto locate_direct = [&](int tile) __attribute__((always_inline)) -> uint32_t {
    if (kWaves > kLoadWaves && wave >= kLoadWaves) return 0u;
    return group_entry(tile, wave);
  };
  auto locate = [&](int tile) __attribute__((always_inline)) -> uint32_t {
    if (kWaves > kLoadWaves && wave >= kLoadWaves) return 0u;
    if (tile < 2) return group_entry(tile, wave);
    return tile < kGroupTabTiles ? gtab[tile * kLoadWaves + wave] : kEntSlow;
  };
  auto issue_tile = [&](uint32_t ent, int tile, unsigned char* kdst,
                        unsigned char* vdst) __attribute__((always_inline)) {
    if (kWaves > kLoadWaves && wave >= kLoadWaves) return;   // waves 0..3 load
    const uint32_t e = __builtin_amdgcn_readfirstlane(ent);
    if (!(e & kEntSlow)) {
      const int64_t r = static_cast<int64_t>(e & kEntRowMask);
      const bool sp = (e & kEntSpecial) != 0;
      const unsigned char* kb;
      const unsigned char* vb;
      if (FUSED && (e & kEntCur) != 0) {
        kb = f->k_in + r * tok_bytes + h * 128;
        vb = f->v_in + r * tok_bytes + h * 128;
      } else {
        kb = (sp ? pool_special : pool_patch) + r * tok_bytes + h * 128;
        vb = kb + static_cast<int64_t>(sp ? a.special_page : a.patch_page) * tok_bytes;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_global_load_lds(
            kb + lane_off[i], (lds_void*)(kdst + (16 * wave + 8 * i) * kRowBytes), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            vb + lane_off[i], (lds_void*)(vdst + (16 * wave + 8 * i) * kRowBytes), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * wave + 8 * i + (lane >> 3);
      int j = kv_begin + tile * kKvTile + row;
      j = j < kv_end ? j : kv_end - 1;   // rows past the end: any valid token
      const bool sp = j >= patch_tok;
      const int s = j - patch_tok;
      const bool in_tail = sp && s >= sp_head;
      const int jj = !sp ? j : in_tail ? s - sp_head + sp_tail_first : s;
      const int pbase = in_tail ? sp_head_pages : 0;
      const int psize = sp ? a.special_page : a.patch_page;
      const int pi = div_small(jj, psize, sp ? a.inv_special_page : a.inv_patch_page);
      const int slot = jj - pi * psize;
      const int chunk = (lane & 7) ^ swz(row);
      const unsigned char* src;
      const unsigned char* vsrc;
      int in_row = -1;   // fused: the row's k/v row when it belongs to a current frame
      if constexpr (FUSED) {
        if (!sp && pi >= pcut_page) {
          in_row = in_row0 + (f_off_p + pi - pcut_page) * f->tokens_per_frame +
                   f->num_special + slot;
        } else if (sp && s >= s_cut) {
          const int u = s - s_cut;
          const int fr = div_small(u, f->num_special, f->inv_num_special);
          in_row = in_row0 + (f_off_s + fr) * f->tokens_per_frame + (u - fr * f->num_special);
        }
      }
      if (in_row >= 0) {
        const int64_t io = static_cast<int64_t>(in_row) * tok_bytes + h * 128 + chunk * 16;
        src = f->k_in + io;
        vsrc = f->v_in + io;
      } else {
        int page;
        if constexpr (COMPACT)
          page = sp ? (in_tail ? w[kWSpecialTailBase] : w[kWSpecialOff]) + pi : patch_ids[pi];
        else
          page = sp ? special_ids[pbase + pi] : patch_ids[pi];
        const int64_t ko = (static_cast<int64_t>(page) * 2 * psize + slot) * HD;
        src = (sp ? pool_special : pool_patch) +
              (ko + static_cast<int64_t>(h) * 64 + chunk * 8) * 2;
        vsrc = src + static_cast<int64_t>(psize) * HD * 2;
      }
      __builtin_amdgcn_global_load_lds(
          src, (lds_void*)(kdst + (16 * wave + 8 * i) * kRowBytes), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          vsrc, (lds_void*)(vdst + (16 * wave + 8 * i) * kRowBytes), 16, 0, 0);
    }
  };

  // LDS read offsets = a lane part (computed once) + a compile-time part.
  // K fragments: row 32hh + 4j + rl with rl = 8(r16/4) + r16%4, chunk
  // 4kk + g.  V^T fragments: row 32hh + 4hf + rv with rv = 8g + r16/4,
  // bytes 32db + 8(r16%4).  swz(row) reads row bits 1, 3 and 4 only, which
  // come from rl (rv), so every chunk position is a lane constant XOR a
  // compile-time value.
  const int rl = 8 * (r16 >> 2) + (r16 & 3);
  const int ck = g ^ swz(rl);
  const uint32_t k_lane[2] = {static_cast<uint32_t>(rl * kRowBytes + (ck << 4)),
                              static_cast<uint32_t>(rl * kRowBytes + ((ck ^ 4) << 4))};
  const int rv = 8 * g + (r16 >> 2);
  const int cv = ((r16 & 3) >> 1) ^ swz(rv);
  uint32_t v_lane[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    v_lane[db] = static_cast<uint32_t>(rv * kRowBytes + (((2 * db) ^ cv) << 4) + 8 * (r16 & 1));
  const int g8 = 8 * g;

  // One 64-key tile in two 32-key halves.  Each half runs in phases kept
  // apart by scheduling barriers, so that the K fragments, the V fragments
  // and the scores are not all live at once:
  //   1. K fragments, S^T for the 4 main tiles and this wave's tail part;
  //   2. V^T fragments, masking of keys past the end;
  //   3. weights against the running reference max, their lane sums, bf16
  //      packing; the rare redo with the exact max; O^T += V^T P^T.
  auto scores = [&](const unsigned char* ks, int hh, bool tail_here, int tj,
                    f32x4 (&sc)[NQT][2], f32x4& st) {
    bf16x8 kf[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        kf[j][kk] = lds_read16(ks, k_lane[kk] + (32 * hh + 4 * j) * kRowBytes);
    // all first halves of the head dimension, then all second halves: each
    // product accumulates in its own registers, so consecutive MFMAs are
    // independent (one shared temporary would chain them)
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) sc[t][j] = mfma(kf[j][0], qf[t][0], zero4);
    if (tail_here) st = mfma(tj == 0 ? kf[0][0] : kf[1][0], qt_tail[0], zero4);
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) sc[t][j] = mfma(kf[j][1], qf[t][1], sc[t][j]);
    if (tail_here) st = mfma(tj == 0 ? kf[0][1] : kf[1][1], qt_tail[1], st);
  };
  auto mask = [&](int vlim, int tj, f32x4 (&sc)[NQT][2], f32x4& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool m0 = g8 >= vlim - i;
      const bool m1 = g8 >= vlim - 4 - i;
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        if (m0) sc[t][0][i] = -INFINITY;
        if (m1) sc[t][1][i] = -INFINITY;
      }
      if (tj ? m1 : m0) st[i] = -INFINITY;
    }
  };
  // weights of 8 (or 4) scores against reference m: packed bf16 and lane sum
  auto weights8 = [&](const f32x4& s0, const f32x4& s1, float m, bf16x8& pf) {
    const float mc = m * c2;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c2, -mc));
      p[4 + i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c2, -mc));
    }
    const u32x4 pw = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                      pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
    pf = __builtin_bit_cast(bf16x8, pw);
    return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  };
  auto weights4 = [&](const f32x4& s, float m, int tj, bf16x8& pf) {
    const float mc = m * c2;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mc));
    const uint32_t p01 = pack_bf16(p[0], p[1]);
    const uint32_t p23 = pack_bf16(p[2], p[3]);
    const u32x4 pw = tj == 0 ? u32x4{p01, p23, 0u, 0u} : u32x4{0u, 0u, p01, p23};
    pf = __builtin_bit_cast(bf16x8, pw);
    return (p[0] + p[1]) + (p[2] + p[3]);
  };

  bool overflow = false;   // a fast tile's weights outgrew the fixed reference
  // first: tile 0 of a pass, where every reference is still the sentinel
  // and O, l are zero -- the row max is taken before the weights, so the
  // half is not computed twice
  auto compute_tile = [&](const unsigned char* ks, const unsigned char* vs, int tile,
                          bool exact, bool first) __attribute__((always_inline)) {
    const int valid = kv_end - (kv_begin + tile * kKvTile);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh * 32 >= valid) break;
      const bool partial = valid < 32 * hh + 32;
      const int vlim = valid - 32 * hh;   // keys of this half below vlim are real
      // this wave's tail part: key block kb = wave, i.e. half wave/2; its
      // smallest key is 32hh + 4tj -- skip it when that one is past the end
      const int tj = wave & 1;
      const bool tail_here = has_tail && wave < kTailWaves && (wave >> 1) == hh &&
                             32 * hh + 4 * tj < valid;

      // ---- phase 1
      f32x4 sc[NQT][2];
      f32x4 st = zero4;
      // raised priority while the score MFMAs issue: the other wave on the
      // SIMD is then usually in its weights phase and fills the VALU
      __builtin_amdgcn_s_setprio(1);
      scores(ks, hh, tail_here, tj, sc, st);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);

      // ---- phase 2
      bf16x8 vf[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        i16x4 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          part[hf] = lds_read_tr(vs, v_lane[db] + (32 * hh + 4 * hf) * kRowBytes);
        vf[db] = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
      if (partial) mask(vlim, tj, sc, st);
      __builtin_amdgcn_sched_barrier(0);

      // ---- phase 3, fast form: the reference max stays fixed, weights and
      // products tile by tile with no branch, so the products of one query
      // tile overlap the weights of the next; weights that outgrow the
      // reference are caught in the running sums after the last tile
      if (!exact) {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          bf16x8 pft_;
          const float ps_ = weights8(sc[t][0], sc[t][1], m_run[t], pft_);
          l_run[t] += ps_;
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[t][db] = mfma(vf[db], pft_, oacc[t][db]);
        }
        if (tail_here) {
          bf16x8 pft_;
          const float pst_ = weights4(st, mtail, tj, pft_);
          ltail += pst_;
#pragma unroll
          for (int db = 0; db < 4; ++db) otail[db] = mfma(vf[db], pft_, otail[db]);
        }
        // order: the weights of query tile 0, then each product of tile t
        // followed by a share (7 vector instructions) of tile t+1's weights,
        // so this wave's MFMAs run under its own vector work (left to itself
        // the compiler forms every weight first)
        __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
#pragma unroll
        for (int t = 1; t < NQT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // seven VALU
          }
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }

      // ---- phase 3, exact form (the first tile, and the rerun)
      bf16x8 pf[NQT];
      float ps[NQT];
      bf16x8 pft;
      float pst = 0.f;
      bool over = false;
      // the main tiles start in half 0; the tail part of a wave lies in one
      // half only, so in the first tile it always starts where it is
      const bool main_first = first && hh == 0;
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        if (main_first) m_run[t] = fmaxf(m_run[t], row_max(max8(sc[t][0], sc[t][1])));
        ps[t] = weights8(sc[t][0], sc[t][1], m_run[t], pf[t]);
        over = over || !(ps[t] <= kSumLimit);
      }
      if (tail_here) {
        if (first)
          mtail = fmaxf(mtail, row_max(fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]))));
        pst = weights4(st, mtail, tj, pft);
        over = over || !(pst <= kSumLimit);
      }
      if (__any(over)) {
        // redo this half with the exact row max (rare)
        scores(ks, hh, tail_here, tj, sc, st);
        if (partial) mask(vlim, tj, sc, st);
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          const float m_new = fmaxf(m_run[t], row_max(max8(sc[t][0], sc[t][1])));
          const float alpha = __builtin_amdgcn_exp2f((m_run[t] - m_new) * c2);
          m_run[t] = m_new;
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[t][db] *= alpha;
          l_run[t] *= alpha;
          ps[t] = weights8(sc[t][0], sc[t][1], m_new, pf[t]);
        }
        if (tail_here) {
          const float mx = row_max(fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3])));
          const float m_new = fmaxf(mtail, mx);
          const float alpha = __builtin_amdgcn_exp2f((mtail - m_new) * c2);
          mtail = m_new;
#pragma unroll
          for (int db = 0; db < 4; ++db) otail[db] *= alpha;
          ltail *= alpha;
          pst = weights4(st, m_new, tj, pft);
        }
      }
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        l_run[t] += ps[t];
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[t][db] = mfma(vf[db], pf[t], oacc[t][db]);
      }
      if (tail_here) {
        ltail += pst;
#pragma unroll
        for (int db = 0; db < 4; ++db) otail[db] = mfma(vf[db], pft, otail[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The lagged waves: each of their fast tiles starts with the weights and
  // products of the previous tile's second half, from scores and V
  // fragments kept in registers, then does its first half whole and only
  // the scores of its second half.  Without this, the barrier at every tile
  // keeps the two waves of a SIMD in step: both issue their score MFMAs at
  // the same time and then both their vector work.
  bool lag_carry = false;
  f32x4 lag_sc[NQT][2];
  bf16x8 lag_vf[4];
  auto read_vf = [&](const unsigned char* vs, int hh, bf16x8 (&vf)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i16x4 part[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        part[hf] = lds_read_tr(vs, v_lane[db] + (32 * hh + 4 * hf) * kRowBytes);
      vf[db] = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // fast-form weights and products of the main tiles of one half
  auto fast_main = [&](const f32x4 (&sc)[NQT][2], const bf16x8 (&vf)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      bf16x8 pft_;
      l_run[t] += weights8(sc[t][0], sc[t][1], m_run[t], pft_);
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[t][db] = mfma(vf[db], pft_, oacc[t][db]);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
#pragma unroll
    for (int t = 1; t < NQT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto finish_lag = [&]() __attribute__((always_inline)) {
    if (lag_carry) fast_main(lag_sc, lag_vf);
  };
  auto lag_tile = [&](const unsigned char* ks, const unsigned char* vs, int tile)
      __attribute__((always_inline)) {
    finish_lag();
    const int valid = kv_end - (kv_begin + tile * kKvTile);
    {
      f32x4 sc[NQT][2];
      f32x4 st = zero4;   // no tail part here
      __builtin_amdgcn_s_setprio(1);
      scores(ks, 0, false, 0, sc, st);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 vf[4];
      read_vf(vs, 0, vf);
      if (valid < 32) mask(valid, 0, sc, st);
      __builtin_amdgcn_sched_barrier(0);
      fast_main(sc, vf);
    }
    lag_carry = valid > 32;
    if (lag_carry) {
      f32x4 st = zero4;
      __builtin_amdgcn_s_setprio(1);
      scores(ks, 1, false, 0, lag_sc, st);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      read_vf(vs, 1, lag_vf);
      if (valid < 64) mask(valid - 32, 0, lag_sc, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two statically distinct buffer pairs, used alternately (loop unrolled by
  // two), so the compiler can tell the reads of one from the loads into the
  // other and does not wait for the loads in flight before reading.
  // The first tile sets the reference max exactly; the others keep it (fast
  // form).  If any wave's weights outgrew it, the workgroup starts over with
  // the exact form on every tile.  The two forms run in separate loops.
  // Start: the first two tiles' page lookups, then q, then the first tile's
  // loads (the lookup's wait leaves q in flight), then the append copy's
  // loads and the table, all in flight together until the first barrier.
  {
    const uint32_t src0 = locate_direct(0);
    uint32_t src = ntiles > 1 ? locate_direct(1) : 0u;
    __builtin_amdgcn_sched_barrier(0);
    load_all_q();
    __builtin_amdgcn_sched_barrier(0);
    issue_tile(src0, 0, kbuf0, vbuf0);
    __builtin_amdgcn_sched_barrier(0);
    fused_loads();
    fill_table();
    if (tid == 0) vote = 0;
    __syncthreads();   // tile 0, q, the table and the vote flag ready
    fused_stores();   // their loads are done: the barrier waited for them
    if (ntiles > 1) issue_tile(src, 1, kbuf1, vbuf1);
    if (ntiles > 2) src = locate(2);
    compute_tile(kbuf0, vbuf0, 0, true, true);
    if (lagged) {
      // the same barriers as the loop below; these waves load nothing
      for (int tile = 1; tile < ntiles; tile += 2) {
        __syncthreads();
        lag_tile(kbuf1, vbuf1, tile);
        if (tile + 1 >= ntiles) break;
        __syncthreads();
        lag_tile(kbuf0, vbuf0, tile + 1);
      }
      finish_lag();
    } else {
      for (int tile = 1; tile < ntiles; tile += 2) {
        // tile's loads done everywhere; everyone is past tile-1 (other buffer)
        __syncthreads();
        if (tile + 1 < ntiles) issue_tile(src, tile + 1, kbuf0, vbuf0);
        if (tile + 2 < ntiles) src = locate(tile + 2);
        compute_tile(kbuf1, vbuf1, tile, false, false);
        if (tile + 1 >= ntiles) break;
        __syncthreads();
        if (tile + 2 < ntiles) issue_tile(src, tile + 2, kbuf1, vbuf1);
        if (tile + 3 < ntiles) src = locate(tile + 3);
        compute_tile(kbuf0, vbuf0, tile + 1, false, false);
      }
    }
  }
  // Fast tiles are checked once, here: a lane's running sum holds every
  // weight it formed, so a weight above kFixedLimit (or an infinite one)
  // shows in it.
#pragma unroll
  for (int t = 0; t < NQT; ++t) overflow = overflow || !(l_run[t] <= kFixedLimit);
  overflow = overflow || !(ltail <= kFixedLimit);
  // The vote: a wave whose sums overflowed sets the flag; the barrier
  // publishes it and also leaves every wave past its last tile read, so the
  // LDS tiles may be loaded again (the rerun) or reused (the tail merge).
  if (__any(overflow) && lane == 0) vote = 1;
  __syncthreads();
  if (vote != 0) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      m_run[t] = kNoMax;
      l_run[t] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[t][db] = zero4;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) otail[db] = zero4;
    ltail = 0.f;
    mtail = kNoMax;
    uint32_t src = locate(0);
    issue_tile(src, 0, kbuf0, vbuf0);
    if (ntiles > 1) src = locate(1);
    for (int tile = 0; tile < ntiles; tile += 2) {
      __syncthreads();
      if (tile + 1 < ntiles) issue_tile(src, tile + 1, kbuf1, vbuf1);
      if (tile + 2 < ntiles) src = locate(tile + 2);
      compute_tile(kbuf0, vbuf0, tile, true, tile == 0);
      if (tile + 1 >= ntiles) break;
      __syncthreads();
      if (tile + 2 < ntiles) issue_tile(src, tile + 2, kbuf0, vbuf0);
      if (tile + 3 < ntiles) src = locate(tile + 3);
      compute_tile(kbuf1, vbuf1, tile + 1, true, false);
    }
    __syncthreads();   // LDS tiles no longer read
  }

  // ---- epilogue: main tiles
  uint16_t* og = static_cast<uint16_t*>(a.o);
  // max |acc| / l over the row's 64 values (lanes r16 + 16g hold 16 each);
  // every lane of the wave takes part
  auto row_absmax = [&](const f32x4* acc, float l) {
    float mx = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[db][i]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    return mx / l;
  };
  auto store_row = [&](int row, const f32x4* acc, float m, float l, float mx) {
    // row of the block, acc = O^T column of this lane, l = row sum,
    // mx = row_absmax(acc, l) (split partials only)
    const int64_t grow = q_row0 + row;
    if (split < 0) {
      const float inv = 1.f / l;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint2 pv;
        pv.x = pack_bf16(acc[db][0] * inv, acc[db][1] * inv);
        pv.y = pack_bf16(acc[db][2] * inv, acc[db][3] * inv);
        *reinterpret_cast<uint2*>(og + (grow * H + h) * 64 + db * 16 + g * 4) = pv;
      }
      if (g == 0 && a.lse != nullptr) a.lse[grow * H + h] = m * a.sm_scale + __logf(l);
    } else {
      // fp16 of (acc / l) / mx, in [-1, 1]; the record keeps m, l and mx
      const int64_t prow = static_cast<int64_t>(split) * a.part_rows + grow;
      const float k = mx > 0.f ? 1.f / (mx * l) : 0.f;
      uint16_t* dst = a.part_o + (prow * H + h) * 64 + g * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint2 pv;
        pv.x = pack_f16(acc[db][0] * k, acc[db][1] * k);
        pv.y = pack_f16(acc[db][2] * k, acc[db][3] * k);
        *reinterpret_cast<uint2*>(dst + db * 16) = pv;
      }
      if (g == 0)
        *reinterpret_cast<float4*>(a.part_ml + (prow * H + h) * 4) =
            float4{m * a.sm_scale, l, mx, 0.f};
    }
  };
  // ---- epilogue: first merge the four waves' parts of the tail tile in LDS
  // (before any store, so its barriers wait for no store in flight)
  f32x4 tacc[4] = {zero4, zero4, zero4, zero4};
  float tM = 0.f, tL = 1.f;
  if (has_tail) {
    ltail += __shfl_xor(ltail, 16);
    ltail += __shfl_xor(ltail, 32);
    float* tm = reinterpret_cast<float*>(kbuf0);     // [4 waves][16 rows]
    float* tl = tm + 4 * 16;                         // [4][16]
    // [wave][16 rows][64]: waves 0, 1 in vbuf0, waves 2, 3 in vbuf1 (4 KiB each)
    auto to_part = [&](int ww) {
      return reinterpret_cast<float*>(ww < 2 ? vbuf0 : vbuf1) + (ww & 1) * 16 * 64;
    };
    if (g == 0 && wave < kTailWaves) {
      tm[wave * 16 + r16] = mtail;
      tl[wave * 16 + r16] = ltail;
    }
    // a part row holds 16 chunks of 4 floats; chunk c of row r sits at
    // position c ^ r, so the 16 rows of one chunk column fall in distinct
    // banks (a plain 256-byte row stride would put them all in the same ones)
    auto part_off = [&](int db) { return r16 * 64 + (((db * 4 + g) ^ r16) << 2); };
    if (wave < kTailWaves) {
      float* mine = to_part(wave);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *reinterpret_cast<f32x4*>(mine + part_off(db)) = otail[db];
    }
    __syncthreads();
    if (wave == 0) {
      // lane (r16, g) finishes row r16, d = db*16 + g*4 + i, like store_row
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kTailWaves; ++ww) M = fmaxf(M, tm[ww * 16 + r16]);
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < kTailWaves; ++ww) {
        const float wgt = __builtin_amdgcn_exp2f((tm[ww * 16 + r16] - M) * c2);
        L += wgt * tl[ww * 16 + r16];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const f32x4 part = *reinterpret_cast<const f32x4*>(to_part(ww) + part_off(db));
#pragma unroll
          for (int i = 0; i < 4; ++i) tacc[db][i] += wgt * part[i];
        }
      }
      tM = M;
      tL = L;
    }
  }

  // ---- epilogue: stores
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    if (t >= nt) break;
    float l = l_run[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float mx = split >= 0 ? row_absmax(oacc[t], l) : 0.f;
    const int row = (wave + t * kWaves) * kQTileRows + r16;
    if (row < q_rows) store_row(row, oacc[t], m_run[t], l, mx);
  }

  if (has_tail && wave == 0) {
    const float mx = split >= 0 ? row_absmax(tacc, tL) : 0.f;
    const int row = kWaves * NQT * kQTileRows + r16;
    if (row < q_rows) store_row(row, tacc, tM, tL, mx);
  }
}

// Two waves per SIMD either way: two 4-wave workgroups or one 8-wave
// workgroup per compute unit.
template <int W, bool COMPACT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_d64_kernel(AttnArgs a) {
  attn_body<false, W, COMPACT>(a, nullptr);
}

// The plan (work items, page ids) is read from the kernel arguments.
static_assert(offsetof(FusedArgs, data) % 8 == 0, "segments in the plan need 8-byte alignment");
template <int W, bool COMPACT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_fused_kernel(FusedArgs f) {
  AttnArgs a = f.a;
  a.work = f.data + f.off_work;
  a.patch_ids = f.data + f.off_pids;
  a.special_ids = f.data + f.off_sids;
  attn_body<true, W, COMPACT>(a, &f);
}

}  // namespace

int launch_attention_bf16(const AttnArgs& a, int waves, void* stream, void* ev0, void* ev1) {
  const dim3 grid(a.n_items, a.heads);
  if (waves == 8 && a.special_compact != 0)
    launch_timed(attn_bf16_d64_kernel<8, true>, grid, dim3(8 * 64), stream, ev0, ev1, a);
  else if (waves == 8)
    launch_timed(attn_bf16_d64_kernel<8, false>, grid, dim3(8 * 64), stream, ev0, ev1, a);
  else if (a.special_compact != 0)
    launch_timed(attn_bf16_d64_kernel<4, true>, grid, dim3(4 * 64), stream, ev0, ev1, a);
  else
    launch_timed(attn_bf16_d64_kernel<4, false>, grid, dim3(4 * 64), stream, ev0, ev1, a);
  return static_cast<int>(hipGetLastError());
}

int launch_attention_fused(const FusedArgs& f, int waves, void* stream, void* ev0, void* ev1) {
  const dim3 grid(f.a.n_items, f.a.heads);
  if (waves == 8 && f.a.special_compact != 0)
    launch_timed(attn_bf16_fused_kernel<8, true>, grid, dim3(8 * 64), stream, ev0, ev1, f);
  else if (waves == 8)
    launch_timed(attn_bf16_fused_kernel<8, false>, grid, dim3(8 * 64), stream, ev0, ev1, f);
  else if (f.a.special_compact != 0)
    launch_timed(attn_bf16_fused_kernel<4, true>, grid, dim3(4 * 64), stream, ev0, ev1, f);
  else
    launch_timed(attn_bf16_fused_kernel<4, false>, grid, dim3(4 * 64), stream, ev0, ev1, f);
  return static_cast<int>(hipGetLastError());
}

}  // namespace psw
