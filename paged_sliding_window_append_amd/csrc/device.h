// Interface between the host library (capi.cpp) and the HIP kernels
// (kernels.hip).  Plain structs passed by value as kernel arguments; every
// launch function returns a hipError_t value as int (0 = success).
#pragma once

#include <cstddef>
#include <cstdint>

namespace psw {

// ---- append_frame K/V write -------------------------------------------
// One contiguous byte range copied from k or v into a pool.
struct AppendSeg {
  int64_t src_off;   // bytes into k (or v)
  int64_t dst_off;   // bytes into the patch (or special) pool
  int32_t bytes;     // multiple of 16
  int32_t flags;     // bit 0: source is v; bit 1: destination is special pool
};
constexpr int kMaxAppendSegs = 120;
constexpr int kAppendChunk = 4096;   // bytes per workgroup
struct AppendArgs {
  const unsigned char* k;
  const unsigned char* v;
  unsigned char* patch;
  unsigned char* special;
  int32_t nseg;
  int32_t max_chunks;                // grid.x: chunks of the longest segment
  AppendSeg seg[kMaxAppendSegs];
};

// Same copy with the segment list in device memory (the per-frame plan
// carries it, so one upload serves every layer).
struct AppendDevArgs {
  const unsigned char* k;
  const unsigned char* v;
  unsigned char* patch;
  unsigned char* special;
  const AppendSeg* seg;
  int32_t nseg;
  int32_t max_chunks;
};

// ---- table + plan upload (through kernel arguments) -------------------
constexpr int kUploadInts = 960;   // multiple of 4
struct UploadArgs {
  int32_t* dst;
  int32_t n;
  int32_t pad;
  int32_t data[kUploadInts];
};

// ---- append fused with the last chunk of the plan upload ------------------
// Workgroup row y < nseg copies segment y (read from the kernel arguments);
// row y == nseg, column 0, writes the n ints of data to dst.
struct AppendUploadArgs {
  const unsigned char* k;
  const unsigned char* v;
  unsigned char* patch;
  unsigned char* special;
  int32_t* dst;
  int32_t n;
  int32_t seg_off;   // ints into data where the segments start (even)
  int32_t nseg;
  int32_t max_chunks;
  int32_t data[kUploadInts];
};

// ---- attention -----------------------------------------------------------
// Work item: one workgroup (per head) attends q rows [q_row0, q_row0+q_rows)
// of one stream over that stream's visible tokens [kv_begin, kv_end).
constexpr int kWorkInts = 16;
enum WorkField : int {
  kWStream = 0,
  kWQRow0 = 1,       // first global query row
  kWQRows = 2,
  kWKvBegin = 3,
  kWKvEnd = 4,
  kWPatchOff = 5,    // index of the stream's first entry in patch_ids
  kWPatchTok = 6,    // visible patch tokens of the stream (pages * P)
  // Listed special pages: index of the stream's first entry in special_ids,
  // or, in the compact form (AttnArgs::special_compact), the page id of the
  // head's first page; the head's pages are then that id and the next ones,
  // the tail's kWSpecialTailBase and the next ones.
  kWSpecialOff = 7,
  kWSplit = 8,       // partial slot, or -1: write o/lse directly
  // Visible special tokens: the first kWSpecialHead tokens of the listed
  // special pages, then the tail from slot kWSpecialTailFirst of page entry
  // kWSpecialHeadPages (= ceil(head / Ps)).
  kWSpecialHead = 9,
  kWSpecialTailFirst = 10,
  kWSpecialHeadPages = 11,
  // Dense check path: the stream's first row in the dense [token][H][D]
  // arrays (visible tokens of the streams before it), the item's query block
  // index within its stream, and the stream's visible token count.
  kWDenseOff = 12,
  kWQBlock = 13,
  kWKvLen = 14,
  kWSpecialTailBase = 15,   // compact form: page id of the tail's first page
};

// Query tiling of the bf16 kernel: 16-row tiles, 17 per query block (up to
// 272 rows).  Two workgroup shapes (the plan picks one per frame): 4 waves
// each own up to 4 tiles for all keys, two workgroups per compute unit; or
// 8 waves each own up to 2 tiles, one workgroup per compute unit (half the
// KV splits, so half the split partials to write and merge).  The 17th
// "tail" tile is shared by waves 0..3 either way, each taking a quarter of
// every key tile, and waves 0..3 load the key tiles (16 rows each).
constexpr int kQTileRows = 16;
constexpr int kMaxSplits = 64;        // KV splits per work item, at most
constexpr int kMaxQTilesPerBlock = 17;
constexpr int kTailWaves = 4;         // waves sharing the tail tile
constexpr int kLoadWaves = 4;         // waves that load a key tile
constexpr int kKvTile = 64;           // keys per LDS tile
// Key tiles of a work item whose 16-row groups get their source from the
// per-workgroup table in LDS (beyond that, row by row); the plan keeps the
// splits at or below it where the split cap allows.
constexpr int kGroupTabTiles = 1024;
// Rows of a pool (and of k/v) are indexed with 29 bits in that table.
constexpr int64_t kMaxPoolRows = int64_t{1} << 29;

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;                  // may be null
  const void* patch_pool;
  const void* special_pool;
  const int32_t* work;
  const int32_t* patch_ids;
  const int32_t* special_ids;
  // Split partials: per (split, row, head) the output divided by its row
  // sum and by sc = max |O| over d, in fp16 ([-1, 1]), and the record
  // (m * sm_scale, l, sc, 0) in fp32.
  uint16_t* part_o;            // [splits][part_rows][H][D] fp16 bits
  float* part_ml;              // [splits][part_rows][H][4]
  int32_t n_items;
  int32_t heads;
  int32_t head_dim;
  int32_t patch_page;          // P
  int32_t special_page;        // Ps
  int32_t part_rows;           // row stride of the partial buffers
  float sm_scale;
  float inv_patch_page;        // 1 / P
  float inv_special_page;      // 1 / Ps
  uint32_t patch_magic;        // n / P = (mulhi(patch_magic, n) + n) >> patch_shift
  uint32_t special_magic;      // the same for Ps
  int32_t patch_shift;
  int32_t special_shift;
  // 1: every stream's listed special pages are two runs of consecutive ids
  // (head, tail), given by kWSpecialOff and kWSpecialTailBase of the work
  // item, and special_ids is not read; 0: special_ids lists them.
  int32_t special_compact;
};

// ---- append fused into the attention launch ---------------------------------
// The whole per-frame plan travels in the kernel arguments (ints of the
// plan blob: work items, page ids, copy segments and their chunk starts, the
// per-stream cuts below).  Workgroup g copies the 4 KiB chunks g, g + n, ...
// (n workgroups) of the frames' K/V into the pools, the first kFusedCopies of
// them held in registers across its start, and workgroup 0 also writes the blob
// to the workspace for the merge, and the rows of the frames being appended
// are read from k/v, not from the pages the same launch writes.
//
// Per-stream cuts (4 ints at off_fcur + 4 b): the current frames whose patch
// pages are visible are the last ones of the stream's patch list, from list
// entry fc[0] on, frame fc[1] + (entry - fc[0]) of the chunk; the visible
// special tokens from visible index fc[2] on are the current frames' ones,
// frame fc[3] + (index - fc[2]) / Ns, row (index - fc[2]) % Ns of it.
constexpr int kFusedInts = 944;
constexpr int kFusedCopies = 4;
struct FusedArgs {
  AttnArgs a;                  // work, patch_ids, special_ids: set in the kernel
  const unsigned char* k_in;   // the frames' K rows [rows][H][D], rows as q
  const unsigned char* v_in;
  int32_t* ws_blob;            // workspace copy of the blob (merge reads it)
  int32_t blob_n;
  int32_t off_work;
  int32_t off_pids;
  int32_t off_sids;
  int32_t off_qo;
  int32_t off_segs;
  int32_t off_cstart;          // nseg + 1 chunk starts of the segments
  int32_t off_fcur;
  int32_t nseg;
  int32_t total_chunks;
  int32_t tokens_per_frame;    // T
  int32_t num_special;         // Ns
  float inv_num_special;
  int32_t pad;
  int32_t data[kFusedInts];
};
static_assert(sizeof(FusedArgs) <= 4096, "kernel arguments");

// Division by a run-time invariant d >= 1 for 0 <= n < 2^31 (Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", 1994,
// round-up multiplier): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l; the sum
// stays below 2^32 because mulhi(m, n) <= n.
inline void div_magic(uint32_t d, uint32_t* m, int32_t* l) {
  int32_t k = 0;
  while ((uint64_t{1} << k) < d) ++k;
  *l = k;
  *m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << k) - d)) / d + 1);
}

struct MergeArgs {
  void* o;
  float* lse;
  const uint16_t* part_o;      // as in AttnArgs
  const float* part_ml;
  const int32_t* qo_indptr;    // [B+1]
  const int32_t* splits;       // [B] splits per stream
  int32_t num_streams;
  int32_t total_rows;
  int32_t heads;
  int32_t head_dim;
  int32_t part_rows;
  int32_t dtype;               // 0 bf16, 1 fp32
  int32_t max_splits;          // largest entry of splits (picks the lane layout)
};

// Dense float32 check path (dense.hip): the table fields of `t` (pools, work
// items, page ids, page sizes, q, lse, sm_scale, heads, n_items) plus the
// dense K/V rows and the float output.
struct DenseArgs {
  AttnArgs t;
  float* k_dense;     // [sum of visible tokens][H][D]
  float* v_dense;
  float* o;           // [rows][H][D] float
  int32_t dtype;      // of q and the pools: 0 bf16, 1 fp32
};

// Scratch of psw_append_attention_noalloc (scratch.hip): bytes of the
// device array, and the address of the current device's copy (looked up on
// the first call on each device).
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
int scratch_address(void** out);

int device_cu_count(int* out);
int launch_upload(const UploadArgs& a, void* stream);
int launch_append(const AppendArgs& a, void* stream);
int launch_append_dev(const AppendDevArgs& a, void* stream);
int launch_append_upload(const AppendUploadArgs& a, void* stream);
// ev0/ev1: HIP events (or null) recorded at the start and the end of the
// kernel's own dispatch, for kernel timing without extra stream packets.
int launch_attention(const AttnArgs& a, int dtype, int waves, void* stream, void* ev0,
                     void* ev1);
// bf16 attention (attention.hip) with 4- or 8-wave workgroups
int launch_attention_bf16(const AttnArgs& a, int waves, void* stream, void* ev0,
                          void* ev1);
int launch_attention_fused(const FusedArgs& f, int waves, void* stream, void* ev0,
                           void* ev1);
int launch_merge(const MergeArgs& a, void* stream, void* ev0, void* ev1);
int launch_gather_visible(const DenseArgs& d, void* stream);    // dense.hip
int launch_dense_attention(const DenseArgs& d, void* stream);   // dense.hip
const char* hip_error_text(int err);

// HIP events for kernel timing.
int timer_create(void** ev);
int timer_elapsed_ms(void* start, void* stop, float* ms);
int timer_destroy(void* ev);

}  // namespace psw
