// C ABI of the paged two-stream KV cache (declared in include/psw.h).
//
// Host side: configuration checks, per-stream bookkeeping (StreamBook), the
// visible page table, the work plan of the attention kernel, and the
// descriptors of the append copy.  Device work goes through device.h.
#include "psw.h"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "device.h"
#include "page_manager.h"

namespace {

thread_local std::string g_err;

psw_status fail(psw_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

psw_status from_err(psw::Err e, const char* what) {
  switch (e) {
    case psw::Err::ok: return PSW_OK;
    case psw::Err::inval: return fail(PSW_EINVAL, std::string(what) + ": invalid argument");
    case psw::Err::nopage: return fail(PSW_ENOPAGE, std::string(what) + ": no free patch page");
    case psw::Err::special_full: return fail(PSW_ESPECIAL_FULL, std::string(what) + ": special pool full");
    case psw::Err::state: return fail(PSW_ESTATE, std::string(what) + ": not valid in this state");
  }
  return fail(PSW_EINVAL, what);
}

psw_status hip_fail(int err, const char* what) {
  return fail(PSW_EHIP, std::string(what) + ": " + psw::hip_error_text(err));
}

// Default cap on KV splits per work item: the plan only reaches it when a
// launch has little work per head (few heads or streams, many keys).
constexpr int kDefaultSplits = 64;
// Fewest KV tiles a split gets before more splits stop paying for the merge
// (2: the frames before the window fills split their few keys more widely;
// a floor of 1, 2 or 3 measured within 0.1% of one another at 224x224 and
// 0.3-0.5% ahead of 4, 6 measured 0.6% behind).
constexpr int kMinTilesPerSplit = 2;
// Workgroups in flight per compute unit the plan aims for: two 4-wave
// workgroups, or one 8-wave workgroup (two waves per SIMD either way).
constexpr int kWorkgroupsPerCu4 = 2;
constexpr int kWorkgroupsPerCu8 = 1;
// The bf16 plan takes 8-wave workgroups (half as many KV splits, so half the
// split partials to write and merge, for a slower tile loop: each wave reads
// the key tile for 2 query tiles instead of 4) when the 4-wave plan would
// split a stream's keys this many ways or more, i.e. when each split has only
// a few key tiles and its partials weigh most.
constexpr int kEightWaveMinSplits = 16;
// Accelerator complex dies (XCDs) of an MI355X; workgroups are dealt to them
// round-robin.
constexpr int kXcds = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t splits_cap(const psw_config& c) {
  return c.max_kv_splits > 0 ? c.max_kv_splits : kDefaultSplits;
}

// Frames one stream may begin at once (psw_begin_frames); bounds the workspace.
int32_t max_chunk(const psw_config& c) {
  return c.max_frames_per_step > 0 ? c.max_frames_per_step : 1;
}

int32_t qblocks_per_stream(const psw_config& c) {
  const int64_t qt =
      ceil_div(static_cast<int64_t>(max_chunk(c)) * c.tokens_per_frame, psw::kQTileRows);
  return static_cast<int32_t>(ceil_div(qt, psw::kMaxQTilesPerBlock));
}

int64_t elem_bytes(const psw_config& c) { return c.dtype == PSW_BF16 ? 2 : 4; }

// Workspace layout: [ints: table + plan][part_ml][part_o], 256-byte aligned.
struct WsLayout {
  int64_t ints;        // capacity of the int region
  int64_t part_rows;   // rows of the partial buffers (B * T)
  size_t ml_off, o_off, total;
};

int64_t max_work_items(const psw_config& c) {
  return static_cast<int64_t>(c.num_streams) * qblocks_per_stream(c) *
         splits_cap(c);
}

WsLayout ws_layout(const psw_config& c) {
  WsLayout L{};
  const int64_t B = c.num_streams;
  // table, work items, and the append segments of one chunk per stream
  // (per frame at most 2 patch + 2 * (Ns + 1) special segments, 6 ints
  // each, plus alignment), then what the one-launch append + attention
  // adds: the segments' chunk starts and 4 ints per stream
  const int64_t F = max_chunk(c);
  const int64_t max_segs = B * F * (2 + 2 * (c.num_special_tokens + 1));
  // special ids: a stream's head and tail ranges may share a page, which
  // is then listed twice (max_special_pages + 1 entries)
  L.ints = 5 * B + 3 + B * c.max_patch_pages + B * (c.max_special_pages + 1) +
           max_work_items(c) * psw::kWorkInts + max_segs * 6 + 2 + (max_segs + 1) + 4 * B;
  L.part_rows = B * F * c.tokens_per_frame;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  L.ml_off = al(static_cast<size_t>(L.ints) * 4);
  const size_t ml_bytes = static_cast<size_t>(splits_cap(c)) * L.part_rows *
                          c.num_heads * 4 * 4;
  L.o_off = L.ml_off + al(ml_bytes);
  const size_t o_bytes = static_cast<size_t>(splits_cap(c)) * L.part_rows *
                         c.num_heads * c.head_dim * 2;
  L.total = L.o_off + al(o_bytes);
  return L;
}

psw_status check_config(const psw_config* c) {
  if (c == nullptr) return fail(PSW_EINVAL, "config is NULL");
  if (c->num_layers < 1) return fail(PSW_EINVAL, "num_layers must be >= 1");
  if (c->num_streams < 1) return fail(PSW_EINVAL, "num_streams must be >= 1");
  if (c->num_heads < 1) return fail(PSW_EINVAL, "num_heads must be >= 1");
  if (c->head_dim != 64) return fail(PSW_EINVAL, "head_dim must be 64");
  if (c->dtype != PSW_BF16 && c->dtype != PSW_FP32)
    return fail(PSW_EINVAL, "dtype must be PSW_BF16 or PSW_FP32");
  if (c->num_special_tokens < 1)
    return fail(PSW_EINVAL, "num_special_tokens must be >= 1");
  if (c->tokens_per_frame <= c->num_special_tokens)
    return fail(PSW_EINVAL, "tokens_per_frame must exceed num_special_tokens");
  if (c->special_page_size < 1) return fail(PSW_EINVAL, "special_page_size must be >= 1");
  if (c->scale_frames < 0 || c->sliding_window < 0)
    return fail(PSW_EINVAL, "scale_frames and sliding_window must be >= 0");
  if (c->include_scale_frames != 0 && c->include_scale_frames != 1)
    return fail(PSW_EINVAL, "include_scale_frames must be 0 or 1");
  if (c->cross_frame_special != 0 && c->cross_frame_special != 1)
    return fail(PSW_EINVAL, "cross_frame_special must be 0 or 1");
  const int64_t S = c->include_scale_frames ? c->scale_frames : 0;
  if (S == 0 && c->sliding_window == 0 && !c->cross_frame_special)
    return fail(PSW_EINVAL, "no scale frames, no window and no cross-frame specials: "
                            "nothing would be visible");
  if (static_cast<int64_t>(c->max_patch_pages) < S + c->sliding_window + 1)
    return fail(PSW_EINVAL, "max_patch_pages must be >= scale_frames + sliding_window + 1");
  if (c->max_special_pages < 1) return fail(PSW_EINVAL, "max_special_pages must be >= 1");
  if (c->max_kv_splits < 0 || c->max_kv_splits > psw::kMaxSplits)
    return fail(PSW_EINVAL, "max_kv_splits must be in [0, 64]");
  if (!(c->sm_scale >= 0.f) || std::isinf(c->sm_scale))
    return fail(PSW_EINVAL, "sm_scale must be finite and >= 0");
  if (c->max_frames_per_step < 0 || c->max_frames_per_step > 64)
    return fail(PSW_EINVAL, "max_frames_per_step must be in [0, 64]");
  // Every element offset used by the kernels must fit comfortably in int64
  // and every token index in int32.
  const int64_t P = c->tokens_per_frame - c->num_special_tokens;
  const int64_t visible = P * (S + static_cast<int64_t>(c->sliding_window)) +
                          static_cast<int64_t>(c->max_special_pages) * c->special_page_size;
  if (visible >= (int64_t{1} << 24)) return fail(PSW_EINVAL, "visible token count too large");
  const int64_t row = static_cast<int64_t>(c->num_heads) * c->head_dim * elem_bytes(*c);
  if (row % 16 != 0) return fail(PSW_EINVAL, "num_heads * head_dim * element size must be a multiple of 16 bytes");
  // token rows of each pool and of one step's k/v, indexed with 29 bits
  const int64_t Bn = c->num_streams;
  if (Bn * c->max_patch_pages * 2 * P >= psw::kMaxPoolRows ||
      Bn * c->max_special_pages * 2 * c->special_page_size >= psw::kMaxPoolRows ||
      Bn * 64 * c->tokens_per_frame >= psw::kMaxPoolRows)
    return fail(PSW_EINVAL, "pools too large (2^29 token rows at most)");
  return PSW_OK;
}

}  // namespace

// Device workspace seen by one call: the bound workspace (laid out by
// ws_layout for the configuration's largest plan) or the library's own
// scratch array (laid out for the current plan only).
struct WsView {
  unsigned char* base = nullptr;
  size_t ml_off = 0, o_off = 0;   // split records and split outputs
  int64_t part_rows = 0;          // row stride of the split buffers
};

struct psw_cache {
  psw_config cfg{};
  int32_t P = 0;
  float sm_scale = 0.f;
  WsLayout ws{};
  std::vector<psw::StreamBook> books;
  std::vector<void*> patch_pool, special_pool;
  WsView bound;                   // the caller's workspace (psw_bind_workspace)
  const WsView* tgt = &bound;     // where this call's device work goes

  // last built (or set) table, host
  bool have_table = false;
  bool table_built = false;   // by psw_build_visible_page_table (not set by the caller)
  std::vector<int32_t> qo, pind, sind, last, pids, sids;
  std::vector<int32_t> shead, stfirst, stlen;   // visible specials: head, tail
  std::vector<int64_t> kv_indptr;              // [B+1] visible tokens, last plan

  // plan (device copy in the workspace)
  bool planned = false;
  int32_t n_items = 0;
  int32_t max_split_used = 0;
  int32_t off_qo = 0, off_splits = 0, off_pids = 0, off_sids = 0, off_work = 0;
  std::vector<int32_t> blob;
  std::vector<int32_t> stream_splits;
  // append segments of the planned frame, in the workspace (-1: none)
  int32_t off_segs = 0, n_segs = -1, seg_max_chunks = 0;
  // the planned blob waits on the host until the next device call
  bool upload_pending = false;
  // fused append + attention: chunk starts of the segments and per-stream
  // cuts in the blob (valid when fused_ok)
  bool fused_ok = false;
  int32_t off_cstart = 0, off_fcur = 0, total_chunks = 0;
  int64_t plan_scores = 0;   // sum over streams of query rows * visible tokens * heads
  int32_t waves = 4;         // workgroup shape of the bf16 kernels (4 or 8 waves)
  // the plan gives every stream's special pages as two runs of consecutive
  // ids (AttnArgs::special_compact); sp_base: per stream, head and tail base
  bool special_compact = false;
  std::vector<int32_t> sp_base;
  int cus = 0;

  // kernel timing: event pairs reused across reads
  bool profiling = false;
  struct Timer {
    std::vector<std::pair<void*, void*>> ev;
    size_t used = 0;
  } t_attn, t_merge;

  ~psw_cache() {
    for (Timer* t : {&t_attn, &t_merge})
      for (auto& pr : t->ev) {
        psw::timer_destroy(pr.first);
        psw::timer_destroy(pr.second);
      }
  }
};

namespace {

// The next timing slot (an event pair, created on first use), or nullptr
// when timing is off.  The launch records both events.
std::pair<void*, void*>* timer_slot(psw_cache* c, psw_cache::Timer* t, int* err) {
  *err = 0;
  if (!c->profiling) return nullptr;
  if (t->used == t->ev.size()) {
    void* a = nullptr;
    void* b = nullptr;
    *err = psw::timer_create(&a);
    if (*err == 0) *err = psw::timer_create(&b);
    if (*err != 0) return nullptr;
    t->ev.emplace_back(a, b);
  }
  return &t->ev[t->used++];
}

}  // namespace

extern "C" {

const char* psw_last_error(void) { return g_err.c_str(); }

psw_status psw_config_check(const psw_config* cfg) { return check_config(cfg); }

psw_status psw_pool_bytes(const psw_config* cfg, size_t* patch, size_t* special,
                          size_t* workspace) {
  psw_status st = check_config(cfg);
  if (st != PSW_OK) return st;
  const size_t row = static_cast<size_t>(cfg->num_heads) * cfg->head_dim * elem_bytes(*cfg);
  const size_t P = static_cast<size_t>(cfg->tokens_per_frame - cfg->num_special_tokens);
  if (patch) *patch = static_cast<size_t>(cfg->num_streams) * cfg->max_patch_pages * 2 * P * row;
  if (special)
    *special = static_cast<size_t>(cfg->num_streams) * cfg->max_special_pages * 2 *
               cfg->special_page_size * row;
  if (workspace) *workspace = ws_layout(*cfg).total;
  return PSW_OK;
}

psw_status psw_create(const psw_config* cfg, psw_cache** out) {
  if (out == nullptr) return fail(PSW_EINVAL, "out is NULL");
  psw_status st = check_config(cfg);
  if (st != PSW_OK) return st;
  psw_cache* c = new psw_cache();
  c->cfg = *cfg;
  c->P = cfg->tokens_per_frame - cfg->num_special_tokens;
  c->sm_scale = cfg->sm_scale > 0.f ? cfg->sm_scale
                                    : 1.0f / std::sqrt(static_cast<float>(cfg->head_dim));
  c->ws = ws_layout(*cfg);
  psw::StreamConfig sc{cfg->include_scale_frames ? cfg->scale_frames : 0,
                       cfg->sliding_window,
                       cfg->num_special_tokens,
                       cfg->special_page_size,
                       cfg->max_patch_pages,
                       cfg->max_special_pages,
                       cfg->cross_frame_special};
  c->books.resize(static_cast<size_t>(cfg->num_streams));
  for (auto& b : c->books) {
    if (b.init(sc) != psw::Err::ok) {
      delete c;
      return fail(PSW_EINVAL, "stream configuration rejected");
    }
  }
  c->patch_pool.assign(static_cast<size_t>(cfg->num_layers), nullptr);
  c->special_pool.assign(static_cast<size_t>(cfg->num_layers), nullptr);
  c->stream_splits.assign(static_cast<size_t>(cfg->num_streams), 1);
  *out = c;
  g_err.clear();
  return PSW_OK;
}

void psw_destroy(psw_cache* c) { delete c; }

#define PSW_CHECK_CACHE(c) \
  if ((c) == nullptr) return fail(PSW_EINVAL, "cache is NULL")
#define PSW_CHECK_STREAM(c, s)                                   \
  if ((s) < 0 || (s) >= (c)->cfg.num_streams)                    \
  return fail(PSW_EINVAL, "stream index out of range")
#define PSW_CHECK_LAYER(c, l)                                    \
  if ((l) < 0 || (l) >= (c)->cfg.num_layers)                     \
  return fail(PSW_EINVAL, "layer index out of range")

static bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

psw_status psw_bind_layer(psw_cache* c, int32_t layer, void* patch_pool, void* special_pool) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (patch_pool == nullptr || special_pool == nullptr)
    return fail(PSW_EINVAL, "pool pointer is NULL");
  if (!aligned16(patch_pool) || !aligned16(special_pool))
    return fail(PSW_EINVAL, "pool pointers must be 16-byte aligned");
  c->patch_pool[static_cast<size_t>(layer)] = patch_pool;
  c->special_pool[static_cast<size_t>(layer)] = special_pool;
  return PSW_OK;
}

psw_status psw_bind_workspace(psw_cache* c, void* ws, size_t bytes) {
  PSW_CHECK_CACHE(c);
  if (ws == nullptr) return fail(PSW_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(PSW_EINVAL, "workspace must be 256-byte aligned");
  if (bytes < c->ws.total) return fail(PSW_EINVAL, "workspace too small");
  c->bound.base = static_cast<unsigned char*>(ws);
  c->bound.ml_off = c->ws.ml_off;
  c->bound.o_off = c->ws.o_off;
  c->bound.part_rows = c->ws.part_rows;
  c->planned = false;
  return PSW_OK;
}

psw_status psw_reset(psw_cache* c, int32_t stream) {
  PSW_CHECK_CACHE(c);
  if (stream < -1 || stream >= c->cfg.num_streams)
    return fail(PSW_EINVAL, "stream index out of range");
  for (int32_t b = 0; b < c->cfg.num_streams; ++b)
    if (stream < 0 || stream == b) c->books[static_cast<size_t>(b)].reset();
  c->have_table = false;
  c->planned = false;
  return PSW_OK;
}

psw_status psw_begin_frame(psw_cache* c, int32_t stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  return from_err(c->books[static_cast<size_t>(stream)].begin_frame(), "begin_frame");
}

psw_status psw_begin_frames(psw_cache* c, int32_t stream, int32_t n) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  if (n < 1 || n > max_chunk(c->cfg))
    return fail(PSW_EINVAL, "frame count must be in [1, max_frames_per_step]");
  return from_err(c->books[static_cast<size_t>(stream)].begin_frames(n), "begin_frames");
}

psw_status psw_evict_frames(psw_cache* c, int32_t stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  return from_err(c->books[static_cast<size_t>(stream)].evict(nullptr), "evict_frames");
}

psw_status psw_set_defer_eviction(psw_cache* c, int32_t stream, int32_t on) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  c->books[static_cast<size_t>(stream)].set_defer(on != 0);
  return PSW_OK;
}

psw_status psw_execute_deferred_eviction(psw_cache* c, int32_t stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  return from_err(c->books[static_cast<size_t>(stream)].execute_deferred_eviction(nullptr),
                  "execute_deferred_eviction");
}

psw_status psw_rollback_last_frame(psw_cache* c, int32_t stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  return from_err(c->books[static_cast<size_t>(stream)].rollback_last_frame(),
                  "rollback_last_frame");
}

psw_status psw_get_cache_stats(psw_cache* c, int32_t stream, psw_stats* out) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  if (out == nullptr) return fail(PSW_EINVAL, "out is NULL");
  const auto& b = c->books[static_cast<size_t>(stream)];
  out->frame_count = b.frame_count();
  out->scale_pages = b.scale_pages();
  out->live_pages = b.live_pages();
  out->free_pages = b.free_pages();
  out->special_tokens = b.special_tokens();
  return PSW_OK;
}

psw_status psw_export_free_list(psw_cache* c, int32_t stream, int32_t* buf, int32_t cap,
                                int32_t* n) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_STREAM(c, stream);
  if (n == nullptr) return fail(PSW_EINVAL, "n is NULL");
  const auto& fs = c->books[static_cast<size_t>(stream)].free_stack();
  *n = static_cast<int32_t>(fs.size());
  if (cap > 0 && buf == nullptr) return fail(PSW_EINVAL, "buf is NULL");
  const int32_t base = stream * c->cfg.max_patch_pages;
  for (int32_t i = 0; i < cap && i < *n; ++i) buf[i] = base + fs[static_cast<size_t>(i)];
  return PSW_OK;
}

// ---- visible page table ------------------------------------------------

psw_status psw_build_visible_page_table(psw_cache* c) {
  PSW_CHECK_CACHE(c);
  const int32_t B = c->cfg.num_streams;
  const int32_t Ps = c->cfg.special_page_size;
  c->qo.assign(1, 0);
  c->pind.assign(1, 0);
  c->sind.assign(1, 0);
  c->last.clear();
  c->pids.clear();
  c->sids.clear();
  c->shead.clear();
  c->stfirst.clear();
  c->stlen.clear();
  for (int32_t b = 0; b < B; ++b) {
    const auto& bk = c->books[static_cast<size_t>(b)];
    int32_t head = 0, t0 = 0, t1 = 0;
    if (bk.has_current()) {
      bk.visible_patch_pages(&c->pids, b * c->cfg.max_patch_pages);
      bk.visible_special_segments(&head, &t0, &t1);
      const int32_t base = b * c->cfg.max_special_pages;
      for (int32_t i = 0; i < (head + Ps - 1) / Ps; ++i) c->sids.push_back(base + i);
      if (t1 > t0)
        for (int32_t i = t0 / Ps; i < (t1 + Ps - 1) / Ps; ++i) c->sids.push_back(base + i);
      c->qo.push_back(c->qo.back() + bk.current_frames() * c->cfg.tokens_per_frame);
    } else {
      c->qo.push_back(c->qo.back());
    }
    const int32_t end = t1 > t0 ? t1 : head;   // position after the last token
    c->last.push_back(end > 0 ? end - ((end + Ps - 1) / Ps - 1) * Ps : 0);
    c->shead.push_back(head);
    c->stfirst.push_back(t1 > t0 ? t0 % Ps : 0);
    c->stlen.push_back(t1 - t0);
    c->pind.push_back(static_cast<int32_t>(c->pids.size()));
    c->sind.push_back(static_cast<int32_t>(c->sids.size()));
  }
  c->have_table = true;
  c->table_built = true;
  c->planned = false;
  return PSW_OK;
}

psw_status psw_get_page_table(psw_cache* c, psw_page_table* out) {
  PSW_CHECK_CACHE(c);
  if (out == nullptr) return fail(PSW_EINVAL, "out is NULL");
  if (!c->have_table) return fail(PSW_ESTATE, "no page table built");
  out->num_streams = c->cfg.num_streams;
  out->qo_indptr = c->qo.data();
  out->patch_indptr = c->pind.data();
  out->patch_ids = c->pids.data();
  out->special_indptr = c->sind.data();
  out->special_ids = c->sids.data();
  out->special_last_len = c->last.data();
  out->special_head_len = c->shead.data();
  out->special_tail_first = c->stfirst.data();
  out->special_tail_len = c->stlen.data();
  return PSW_OK;
}

psw_status psw_set_page_table(psw_cache* c, const psw_page_table* t) {
  PSW_CHECK_CACHE(c);
  if (t == nullptr || t->qo_indptr == nullptr || t->patch_indptr == nullptr ||
      t->special_indptr == nullptr || t->special_last_len == nullptr)
    return fail(PSW_EINVAL, "table pointer is NULL");
  const psw_config& cf = c->cfg;
  const int32_t B = cf.num_streams;
  if (t->num_streams != B) return fail(PSW_EINVAL, "table has the wrong number of streams");
  const bool has_segments = t->special_head_len != nullptr && t->special_tail_first != nullptr &&
                            t->special_tail_len != nullptr;
  if (!has_segments && (t->special_head_len != nullptr || t->special_tail_first != nullptr ||
                        t->special_tail_len != nullptr))
    return fail(PSW_EINVAL, "special head/tail arrays: give all three or none");
  if (t->qo_indptr[0] != 0 || t->patch_indptr[0] != 0 || t->special_indptr[0] != 0)
    return fail(PSW_EINVAL, "indptr must start at 0");
  for (int32_t b = 0; b < B; ++b) {
    const int32_t nq = t->qo_indptr[b + 1] - t->qo_indptr[b];
    const int32_t np = t->patch_indptr[b + 1] - t->patch_indptr[b];
    const int32_t ns = t->special_indptr[b + 1] - t->special_indptr[b];
    if (nq < 0 || nq % cf.tokens_per_frame != 0 ||
        nq / cf.tokens_per_frame > max_chunk(cf))
      return fail(PSW_EINVAL,
                  "qo length must be k * tokens_per_frame, 0 <= k <= max_frames_per_step");
    // with head and tail ranges, the page where the head ends may also be
    // where the tail starts: listed twice
    if (np < 0 || np > cf.max_patch_pages || ns < 0 ||
        ns > cf.max_special_pages + (has_segments ? 1 : 0))
      return fail(PSW_EINVAL, "page count out of range");
    if (nq > 0 && np == 0 && ns == 0) return fail(PSW_EINVAL, "stream with queries has no pages");
    if (ns > 0 && (t->special_last_len[b] < 1 || t->special_last_len[b] > cf.special_page_size))
      return fail(PSW_EINVAL, "special_last_len out of range");
    if (has_segments) {
      // the listed pages must be exactly the head's and the tail's
      const int32_t Ps = cf.special_page_size;
      const int32_t h = t->special_head_len[b], f = t->special_tail_first[b],
                    n = t->special_tail_len[b];
      if (h < 0 || n < 0 || f < 0 || f >= Ps || (n == 0 && f != 0))
        return fail(PSW_EINVAL, "special head/tail out of range");
      const int32_t hp = (h + Ps - 1) / Ps, tp = (f + n + Ps - 1) / Ps;
      if (hp + tp != ns) return fail(PSW_EINVAL, "special head/tail do not match the pages");
      const int32_t end = n > 0 ? f + n : h;
      if (ns > 0 && t->special_last_len[b] != end - ((end + Ps - 1) / Ps - 1) * Ps)
        return fail(PSW_EINVAL, "special_last_len does not match the head/tail");
    }
    if ((np > 0 && t->patch_ids == nullptr) || (ns > 0 && t->special_ids == nullptr))
      return fail(PSW_EINVAL, "page id array is NULL");
    for (int32_t i = t->patch_indptr[b]; i < t->patch_indptr[b + 1]; ++i) {
      const int32_t p = t->patch_ids[i];
      if (p < b * cf.max_patch_pages || p >= (b + 1) * cf.max_patch_pages)
        return fail(PSW_EINVAL, "patch page id outside the stream's range");
    }
    for (int32_t i = t->special_indptr[b]; i < t->special_indptr[b + 1]; ++i) {
      const int32_t p = t->special_ids[i];
      if (p < b * cf.max_special_pages || p >= (b + 1) * cf.max_special_pages)
        return fail(PSW_EINVAL, "special page id outside the stream's range");
    }
  }
  c->qo.assign(t->qo_indptr, t->qo_indptr + B + 1);
  c->pind.assign(t->patch_indptr, t->patch_indptr + B + 1);
  c->sind.assign(t->special_indptr, t->special_indptr + B + 1);
  c->last.assign(t->special_last_len, t->special_last_len + B);
  if (has_segments) {
    c->shead.assign(t->special_head_len, t->special_head_len + B);
    c->stfirst.assign(t->special_tail_first, t->special_tail_first + B);
    c->stlen.assign(t->special_tail_len, t->special_tail_len + B);
  } else {
    // every listed special token is visible: all in the head
    c->shead.assign(static_cast<size_t>(B), 0);
    c->stfirst.assign(static_cast<size_t>(B), 0);
    c->stlen.assign(static_cast<size_t>(B), 0);
    for (int32_t b = 0; b < B; ++b) {
      const int32_t ns = t->special_indptr[b + 1] - t->special_indptr[b];
      c->shead[static_cast<size_t>(b)] =
          ns > 0 ? (ns - 1) * cf.special_page_size + t->special_last_len[b] : 0;
    }
  }
  c->pids.assign(t->patch_ids ? t->patch_ids : c->pids.data(),
                 t->patch_ids ? t->patch_ids + t->patch_indptr[B] : c->pids.data());
  c->sids.assign(t->special_ids ? t->special_ids : c->sids.data(),
                 t->special_ids ? t->special_ids + t->special_indptr[B] : c->sids.data());
  c->have_table = true;
  c->table_built = false;
  c->planned = false;
  return PSW_OK;
}

static psw_status frame_segments(psw_cache* c, int32_t b, int64_t src_row0,
                                 std::vector<psw::AppendSeg>* segs);

// ---- plan -------------------------------------------------------------------

// Copies ints [from, to) of the planned blob to the workspace through kernel
// arguments, kUploadInts per launch.
static psw_status upload_range(psw_cache* c, size_t from, size_t to, void* stream) {
  int32_t* dst = reinterpret_cast<int32_t*>(c->tgt->base);
  for (size_t off = from; off < to; off += psw::kUploadInts) {
    psw::UploadArgs ua{};
    ua.dst = dst + off;
    ua.n = static_cast<int32_t>(std::min<size_t>(psw::kUploadInts, to - off));
    std::memcpy(ua.data, c->blob.data() + off, static_cast<size_t>(ua.n) * 4);
    const int e = psw::launch_upload(ua, stream);
    if (e != 0) return hip_fail(e, "plan: upload");
  }
  return PSW_OK;
}

// Writes a pending plan to the device on `stream` (before any kernel that
// reads it).
static psw_status flush_plan(psw_cache* c, void* stream) {
  if (!c->upload_pending) return PSW_OK;
  const psw_status st = upload_range(c, 0, c->blob.size(), stream);
  if (st == PSW_OK) c->upload_pending = false;
  return st;
}

// Start of the blob's last upload chunk; the append of the frame can carry
// that chunk when its segments lie inside it.
static size_t last_chunk_start(const psw_cache* c) {
  const size_t n = c->blob.size();
  return n > static_cast<size_t>(psw::kUploadInts) ? n - psw::kUploadInts : 0;
}

// Appends to the blob what the fused append + attention launch needs beyond
// the plan: the chunk starts of the copy segments and, per stream, where the
// current frames' rows begin in the visible order (see FusedArgs).  False
// when the visible current rows are not such a suffix (then the fused entry
// point runs the append and the attention as two launches).
static bool fused_cuts(psw_cache* c) {
  std::vector<int32_t>& blob = c->blob;
  const psw_config& cf = c->cfg;
  const int32_t B = cf.num_streams, Ps = cf.special_page_size, Ns = cf.num_special_tokens;
  c->off_cstart = static_cast<int32_t>(blob.size());
  const auto* segs = reinterpret_cast<const psw::AppendSeg*>(blob.data() + c->off_segs);
  std::vector<int32_t> cstart(1, 0);
  for (int32_t i = 0; i < c->n_segs; ++i)
    cstart.push_back(cstart.back() +
                     static_cast<int32_t>(ceil_div(segs[i].bytes, psw::kAppendChunk)));
  c->total_chunks = cstart.back();
  blob.insert(blob.end(), cstart.begin(), cstart.end());
  c->off_fcur = static_cast<int32_t>(blob.size());
  blob.resize(blob.size() + 4 * static_cast<size_t>(B), 0);
  for (int32_t b = 0; b < B; ++b) {
    if (c->qo[b + 1] == c->qo[b]) continue;
    const auto& bk = c->books[static_cast<size_t>(b)];
    const int32_t F = bk.current_frames();
    const int32_t p0 = c->pind[b], np = c->pind[b + 1] - p0;
    const int32_t pbase = b * cf.max_patch_pages;
    // patch pages: the current frames listed last, in frame order
    int32_t fv = 0;
    while (fv < F && fv < np &&
           c->pids[static_cast<size_t>(p0 + np - 1 - fv)] == pbase + bk.current_page(F - 1 - fv))
      ++fv;
    for (int32_t i = 0; i < np - fv; ++i)
      for (int32_t f = 0; f < F; ++f)
        if (c->pids[static_cast<size_t>(p0 + i)] == pbase + bk.current_page(f)) return false;
    // special tokens: visible positions are [0, head) then [t0, t0 + tl);
    // the current frames own [n0, n0 + F Ns)
    const int32_t head = c->shead[static_cast<size_t>(b)], tl = c->stlen[static_cast<size_t>(b)];
    const int32_t n0 = bk.current_special_start();
    int32_t t0 = 0;
    if (tl > 0) {
      const int32_t hp = (head + Ps - 1) / Ps;
      t0 = (c->sids[static_cast<size_t>(c->sind[b] + hp)] - b * cf.max_special_pages) * Ps +
           c->stfirst[static_cast<size_t>(b)];
    }
    int32_t s_cut, pos_cut;
    if (head > n0) {
      if (tl > 0 && t0 != head) return false;   // not one run of positions
      s_cut = n0;
      pos_cut = n0;
    } else if (tl > 0 && t0 + tl > n0) {
      s_cut = head + std::max(0, n0 - t0);
      pos_cut = std::max(n0, t0);
    } else {
      s_cut = head + tl;   // none visible
      pos_cut = n0;
    }
    if ((pos_cut - n0) % Ns != 0) return false;
    int32_t* fc = blob.data() + c->off_fcur + 4 * b;
    fc[0] = np - fv;
    fc[1] = F - fv;
    fc[2] = s_cut;
    fc[3] = (pos_cut - n0) / Ns;
  }
  return true;
}

// The plan of the current table.  compact: give the special pages as two
// runs of consecutive ids per stream where the table allows it (see below).
static psw_status plan_impl(psw_cache* c, bool compact) {
  const psw_config& cf = c->cfg;
  const int32_t B = cf.num_streams;
  if (c->cus <= 0) {
    int cus = 0;
    const int e = psw::device_cu_count(&cus);
    if (e != 0) return hip_fail(e, "plan: device query");
    c->cus = cus > 0 ? cus : 1;
  }
  // per-stream visible token counts and query blocks
  std::vector<int64_t> kv_len(static_cast<size_t>(B), 0);
  std::vector<int32_t> nqb(static_cast<size_t>(B), 0);
  int64_t work_units = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t nq = c->qo[b + 1] - c->qo[b];
    if (nq == 0) continue;
    const int64_t np = c->pind[b + 1] - c->pind[b];
    kv_len[b] = np * c->P + c->shead[static_cast<size_t>(b)] + c->stlen[static_cast<size_t>(b)];
    const int64_t qt = ceil_div(nq, psw::kQTileRows);
    nqb[b] = static_cast<int32_t>(ceil_div(qt, psw::kMaxQTilesPerBlock));
    work_units += nqb[b] * ceil_div(kv_len[b], psw::kKvTile);
  }
  const int32_t cap = splits_cap(cf);
  // key tiles per split for `per_cu` workgroups per compute unit, and the
  // most splits any stream then gets
  auto chunk_for = [&](int per_cu) {
    const int64_t target = static_cast<int64_t>(c->cus) * per_cu;
    return std::max<int64_t>(kMinTilesPerSplit,
                             ceil_div(work_units * cf.num_heads, std::max<int64_t>(target, 1)));
  };
  auto max_splits_for = [&](int64_t chunk) {
    int64_t m = 0;
    for (int32_t b = 0; b < B; ++b)
      if (nqb[b] > 0)
        m = std::max(m, std::min<int64_t>(cap, ceil_div(ceil_div(kv_len[b], psw::kKvTile), chunk)));
    return m;
  };
  int64_t chunk = chunk_for(kWorkgroupsPerCu4);
  c->waves = 4;
  if (cf.dtype == PSW_BF16 && max_splits_for(chunk) >= kEightWaveMinSplits) {
    chunk = chunk_for(kWorkgroupsPerCu8);
    c->waves = 8;
  }

  // Special pages in the compact form (when asked for) if every stream's
  // list is a head run and a tail run of consecutive page ids (always so for
  // a table built by psw_build_visible_page_table; a caller's table may
  // differ): the plan then carries two base ids per stream instead of the
  // list, so its size does not grow with the special pages a long video has
  // listed.
  c->special_compact = compact;
  c->sp_base.assign(2 * static_cast<size_t>(B), 0);
  for (int32_t b = 0; b < B && c->special_compact; ++b) {
    const int32_t s0 = c->sind[b], n = c->sind[b + 1] - c->sind[b];
    const int32_t hp = std::min(
        n, (c->shead[static_cast<size_t>(b)] + cf.special_page_size - 1) / cf.special_page_size);
    for (int32_t i = 0; i < n && c->special_compact; ++i) {
      const int32_t run0 = i < hp ? 0 : hp;   // first entry of this entry's run
      if (c->sids[static_cast<size_t>(s0 + i)] != c->sids[static_cast<size_t>(s0 + run0)] + (i - run0))
        c->special_compact = false;
    }
    if (hp > 0) c->sp_base[2 * static_cast<size_t>(b)] = c->sids[static_cast<size_t>(s0)];
    if (n > hp) c->sp_base[2 * static_cast<size_t>(b) + 1] = c->sids[static_cast<size_t>(s0 + hp)];
  }

  // compact blob: qo | splits | pind | sind | last | pids | sids | work
  // (sids empty in the compact form)
  std::vector<int32_t>& blob = c->blob;
  blob.clear();
  c->off_qo = 0;
  blob.insert(blob.end(), c->qo.begin(), c->qo.end());
  c->off_splits = static_cast<int32_t>(blob.size());
  blob.resize(blob.size() + static_cast<size_t>(B), 1);
  blob.insert(blob.end(), c->pind.begin(), c->pind.end());
  blob.insert(blob.end(), c->sind.begin(), c->sind.end());
  blob.insert(blob.end(), c->last.begin(), c->last.end());
  c->off_pids = static_cast<int32_t>(blob.size());
  blob.insert(blob.end(), c->pids.begin(), c->pids.end());
  c->off_sids = static_cast<int32_t>(blob.size());
  if (!c->special_compact) blob.insert(blob.end(), c->sids.begin(), c->sids.end());
  c->off_work = static_cast<int32_t>(blob.size());

  // dense row offsets of the streams' visible tokens (the dense check path)
  std::vector<int64_t> kv_ptr(static_cast<size_t>(B) + 1, 0);
  for (int32_t b = 0; b < B; ++b) kv_ptr[b + 1] = kv_ptr[b] + kv_len[b];
  if (kv_ptr[B] > INT32_MAX) return fail(PSW_EINVAL, "too many visible tokens");

  int32_t items = 0;
  int32_t max_split = 0;
  std::vector<std::array<int32_t, psw::kWorkInts>> work;
  std::vector<int32_t> group;   // (stream, split) group of each item
  int64_t ngroups = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t nq = c->qo[b + 1] - c->qo[b];
    if (nq == 0) {
      c->stream_splits[static_cast<size_t>(b)] = 1;
      continue;
    }
    const int64_t kvt = ceil_div(kv_len[b], psw::kKvTile);
    // at most kGroupTabTiles key tiles per split where the cap allows
    int32_t ns = static_cast<int32_t>(std::min<int64_t>(
        cap, std::max(ceil_div(kvt, chunk), ceil_div(kvt, psw::kGroupTabTiles))));
    if (cf.dtype != PSW_BF16) ns = 1;
    ns = std::max(ns, 1);
    c->stream_splits[static_cast<size_t>(b)] = ns;
    blob[static_cast<size_t>(c->off_splits + b)] = ns;
    max_split = std::max(max_split, ns);
    const int64_t qt = ceil_div(nq, psw::kQTileRows);
    for (int32_t qb = 0; qb < nqb[b]; ++qb) {
      const int64_t t0 = qt * qb / nqb[b], t1 = qt * (qb + 1) / nqb[b];
      const int32_t r0 = static_cast<int32_t>(t0 * psw::kQTileRows);
      const int32_t r1 = static_cast<int32_t>(std::min<int64_t>(t1 * psw::kQTileRows, nq));
      for (int32_t s = 0; s < ns; ++s) {
        const int64_t k0 = kvt * s / ns * psw::kKvTile;
        const int64_t k1 = std::min<int64_t>(kvt * (s + 1) / ns * psw::kKvTile, kv_len[b]);
        int32_t wi[psw::kWorkInts] = {0};
        wi[psw::kWStream] = b;
        wi[psw::kWQRow0] = c->qo[b] + r0;
        wi[psw::kWQRows] = r1 - r0;
        wi[psw::kWKvBegin] = static_cast<int32_t>(k0);
        wi[psw::kWKvEnd] = static_cast<int32_t>(k1);
        wi[psw::kWPatchOff] = c->pind[b];
        wi[psw::kWPatchTok] = (c->pind[b + 1] - c->pind[b]) * c->P;
        wi[psw::kWSpecialOff] =
            c->special_compact ? c->sp_base[2 * static_cast<size_t>(b)] : c->sind[b];
        wi[psw::kWSpecialTailBase] =
            c->special_compact ? c->sp_base[2 * static_cast<size_t>(b) + 1] : 0;
        wi[psw::kWSplit] = ns > 1 ? s : -1;
        const int32_t head = c->shead[static_cast<size_t>(b)];
        wi[psw::kWSpecialHead] = head;
        wi[psw::kWSpecialTailFirst] = c->stfirst[static_cast<size_t>(b)];
        wi[psw::kWSpecialHeadPages] = (head + cf.special_page_size - 1) / cf.special_page_size;
        wi[psw::kWDenseOff] = static_cast<int32_t>(kv_ptr[b]);
        wi[psw::kWQBlock] = qb;
        wi[psw::kWKvLen] = static_cast<int32_t>(kv_len[b]);
        work.emplace_back();
        std::copy(wi, wi + psw::kWorkInts, work.back().begin());
        group.push_back(static_cast<int32_t>(ngroups + s));
      }
    }
    ngroups += ns;
  }
  // XCD placement.  Workgroups go to the 8 XCDs round-robin by linear index
  // (item + n_items * head), so for a given head items whose indices agree
  // mod 8 share an XCD and its L2.  The query blocks of one stream and split
  // read the same K/V: their group gets one residue (the least loaded one),
  // and empty items fill the residues that run short.  An odd item count
  // then moves every group to another XCD from one head to the next, so
  // fewer than 8 groups still spread over all XCDs.
  std::vector<int32_t> order;   // item index per position, -1 = empty item
  if (static_cast<int64_t>(work.size()) > ngroups) {
    std::vector<std::vector<int32_t>> bins(kXcds);
    std::vector<int32_t> bin_of(static_cast<size_t>(ngroups), -1);
    for (size_t i = 0; i < work.size(); ++i) {
      int32_t& bn = bin_of[static_cast<size_t>(group[i])];
      if (bn < 0) {
        bn = 0;
        for (int32_t k = 1; k < kXcds; ++k)
          if (bins[k].size() < bins[static_cast<size_t>(bn)].size()) bn = k;
      }
      bins[static_cast<size_t>(bn)].push_back(static_cast<int32_t>(i));
    }
    size_t rows = 0;
    for (const auto& bv : bins) rows = std::max(rows, bv.size());
    if (static_cast<int64_t>(rows) * kXcds <= max_work_items(cf)) {
      for (size_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < kXcds; ++k)
          order.push_back(r < bins[k].size() ? bins[k][r] : -1);
      while (!order.empty() && order.back() < 0) order.pop_back();
      if (order.size() % 2 == 0 &&
          static_cast<int64_t>(order.size()) + 1 <= max_work_items(cf))
        order.push_back(-1);
    }
  }
  if (order.empty())
    for (size_t i = 0; i < work.size(); ++i) order.push_back(static_cast<int32_t>(i));
  for (int32_t i : order) {
    if (i >= 0) {
      blob.insert(blob.end(), work[static_cast<size_t>(i)].begin(),
                  work[static_cast<size_t>(i)].end());
    } else {   // empty item: no rows, no keys, in no stream's first block
      int32_t wi[psw::kWorkInts] = {0};
      wi[psw::kWSplit] = -1;
      wi[psw::kWQBlock] = -1;
      blob.insert(blob.end(), wi, wi + psw::kWorkInts);
    }
    ++items;
  }
  // append segments of every stream in the table (used by psw_append_frames)
  {
    std::vector<psw::AppendSeg> segs;
    bool ok = true;
    for (int32_t b = 0; b < B && ok; ++b) {
      if (c->qo[b + 1] == c->qo[b]) continue;
      if (!c->books[static_cast<size_t>(b)].has_current()) ok = false;
      else frame_segments(c, b, c->qo[b], &segs);
    }
    if (blob.size() & 1) blob.push_back(0);   // 8-byte alignment of the segments
    c->off_segs = static_cast<int32_t>(blob.size());
    c->n_segs = ok ? static_cast<int32_t>(segs.size()) : -1;
    int64_t maxb = 0;
    if (ok) {
      static_assert(sizeof(psw::AppendSeg) == 6 * sizeof(int32_t), "segment layout");
      const size_t n0 = blob.size();
      blob.resize(n0 + segs.size() * 6);
      std::memcpy(blob.data() + n0, segs.data(), segs.size() * sizeof(psw::AppendSeg));
      for (const auto& sg : segs) maxb = std::max<int64_t>(maxb, sg.bytes);
    }
    c->seg_max_chunks = static_cast<int32_t>(ceil_div(maxb, psw::kAppendChunk));
  }
  c->fused_ok = c->n_segs >= 0 && c->table_built && fused_cuts(c);
  if (static_cast<int64_t>(blob.size()) > c->ws.ints)
    return fail(PSW_EINVAL, "plan does not fit the workspace");
  c->upload_pending = true;
  c->plan_scores = 0;
  for (int32_t b = 0; b < B; ++b)
    c->plan_scores += static_cast<int64_t>(c->qo[b + 1] - c->qo[b]) * kv_len[b] * cf.num_heads;
  c->kv_indptr = std::move(kv_ptr);
  c->n_items = items;
  c->max_split_used = max_split;
  c->planned = true;
  return PSW_OK;
}

psw_status psw_profile_enable(psw_cache* c, int32_t on) {
  PSW_CHECK_CACHE(c);
  c->profiling = on != 0;
  return PSW_OK;
}

psw_status psw_profile_read(psw_cache* c, double* attn_ms, int32_t* attn_n, double* merge_ms,
                            int32_t* merge_n) {
  PSW_CHECK_CACHE(c);
  double sums[2] = {0.0, 0.0};
  int32_t counts[2] = {0, 0};
  psw_cache::Timer* ts[2] = {&c->t_attn, &c->t_merge};
  for (int i = 0; i < 2; ++i) {
    for (size_t j = 0; j < ts[i]->used; ++j) {
      float ms = 0.f;
      const int e = psw::timer_elapsed_ms(ts[i]->ev[j].first, ts[i]->ev[j].second, &ms);
      if (e != 0) return hip_fail(e, "profile_read");
      sums[i] += ms;
    }
    counts[i] = static_cast<int32_t>(ts[i]->used);
    ts[i]->used = 0;
  }
  if (attn_ms) *attn_ms = sums[0];
  if (attn_n) *attn_n = counts[0];
  if (merge_ms) *merge_ms = sums[1];
  if (merge_n) *merge_n = counts[1];
  return PSW_OK;
}

psw_status psw_plan_info(psw_cache* c, int32_t* work_items, int32_t* max_splits_used) {
  PSW_CHECK_CACHE(c);
  if (!c->planned) return fail(PSW_ESTATE, "no plan");
  if (work_items) *work_items = c->n_items;
  if (max_splits_used) *max_splits_used = c->max_split_used;
  return PSW_OK;
}

psw_status psw_plan_waves(psw_cache* c, int32_t* waves) {
  PSW_CHECK_CACHE(c);
  if (waves == nullptr) return fail(PSW_EINVAL, "waves is NULL");
  if (!c->planned) return fail(PSW_ESTATE, "no plan");
  *waves = c->waves;
  return PSW_OK;
}

// ---- append ------------------------------------------------------------------

// Appends the copy segments of stream b's current chunk (source rows start
// at row src_row0 of k/v; frame f of the chunk at src_row0 + f * T) to `segs`.
static psw_status frame_segments(psw_cache* c, int32_t b, int64_t src_row0,
                                 std::vector<psw::AppendSeg>* segs) {
  const auto& bk = c->books[static_cast<size_t>(b)];
  if (!bk.has_current()) return fail(PSW_ESTATE, "stream has no current frame");
  const psw_config& cf = c->cfg;
  const int64_t row = static_cast<int64_t>(cf.num_heads) * cf.head_dim * elem_bytes(cf);
  const int64_t P = c->P, Ps = cf.special_page_size, Ns = cf.num_special_tokens;
  const int64_t T = cf.tokens_per_frame;
  for (int32_t f = 0; f < bk.current_frames(); ++f) {
    const int64_t page = static_cast<int64_t>(b) * cf.max_patch_pages + bk.current_page(f);
    const int64_t r0 = src_row0 + f * T;
    for (int kv = 0; kv < 2; ++kv) {
      // patches: rows [Ns, T) -> slots [0, P) of the frame's patch page
      psw::AppendSeg s{};
      s.src_off = (r0 + Ns) * row;
      s.dst_off = (page * 2 + kv) * P * row;
      s.bytes = static_cast<int32_t>(P * row);
      s.flags = kv;
      segs->push_back(s);
      // specials: rows [0, Ns) -> positions [n0, n0 + Ns), split at page ends
      int64_t pos = bk.current_special_start() + f * Ns;
      int64_t r = 0;
      while (r < Ns) {
        const int64_t sp = pos / Ps, slot = pos % Ps;
        const int64_t n = std::min<int64_t>(Ns - r, Ps - slot);
        const int64_t gpage = static_cast<int64_t>(b) * cf.max_special_pages + sp;
        psw::AppendSeg t{};
        t.src_off = (r0 + r) * row;
        t.dst_off = ((gpage * 2 + kv) * Ps + slot) * row;
        t.bytes = static_cast<int32_t>(n * row);
        t.flags = kv | 2;
        segs->push_back(t);
        r += n;
        pos += n;
      }
    }
  }
  return PSW_OK;
}

static psw_status launch_segments(psw_cache* c, int32_t layer, const void* k, const void* v,
                                  const std::vector<psw::AppendSeg>& segs, void* stream) {
  for (size_t i0 = 0; i0 < segs.size(); i0 += psw::kMaxAppendSegs) {
    psw::AppendArgs a{};
    a.k = static_cast<const unsigned char*>(k);
    a.v = static_cast<const unsigned char*>(v);
    a.patch = static_cast<unsigned char*>(c->patch_pool[static_cast<size_t>(layer)]);
    a.special = static_cast<unsigned char*>(c->special_pool[static_cast<size_t>(layer)]);
    const size_t n = std::min<size_t>(psw::kMaxAppendSegs, segs.size() - i0);
    a.nseg = static_cast<int32_t>(n);
    int64_t maxb = 0;
    for (size_t i = 0; i < n; ++i) {
      a.seg[i] = segs[i0 + i];
      maxb = std::max<int64_t>(maxb, a.seg[i].bytes);
    }
    a.max_chunks = static_cast<int32_t>(ceil_div(maxb, psw::kAppendChunk));
    const int e = psw::launch_append(a, stream);
    if (e != 0) return hip_fail(e, "append");
  }
  return PSW_OK;
}

psw_status psw_append_frame(psw_cache* c, int32_t layer, int32_t stream, const void* k,
                            const void* v, void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  PSW_CHECK_STREAM(c, stream);
  if (k == nullptr || v == nullptr) return fail(PSW_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(PSW_EINVAL, "k and v must be 16-byte aligned");
  if (c->patch_pool[static_cast<size_t>(layer)] == nullptr)
    return fail(PSW_EUNBOUND, "layer pools not bound");
  std::vector<psw::AppendSeg> segs;
  psw_status st = frame_segments(c, stream, 0, &segs);
  if (st != PSW_OK) return st;
  return launch_segments(c, layer, k, v, segs, hip_stream);
}

psw_status psw_append_frames(psw_cache* c, int32_t layer, const void* k, const void* v,
                             void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (c->have_table && c->qo.back() == 0) return PSW_OK;   // no stream has a frame
  if (k == nullptr || v == nullptr) return fail(PSW_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(PSW_EINVAL, "k and v must be 16-byte aligned");
  if (c->patch_pool[static_cast<size_t>(layer)] == nullptr)
    return fail(PSW_EUNBOUND, "layer pools not bound");
  if (!c->have_table) return fail(PSW_ESTATE, "no page table built");
  if (c->planned && c->n_segs >= 0 && c->tgt->base == nullptr)
    return fail(PSW_EUNBOUND, "workspace not bound");
  if (c->planned && c->n_segs >= 0 && c->upload_pending &&
      last_chunk_start(c) <= static_cast<size_t>(c->off_segs)) {
    // the plan's last chunk and the K/V copy in one launch
    const size_t c0 = last_chunk_start(c);
    psw_status st = upload_range(c, 0, c0, hip_stream);
    if (st != PSW_OK) return st;
    psw::AppendUploadArgs a{};
    a.k = static_cast<const unsigned char*>(k);
    a.v = static_cast<const unsigned char*>(v);
    a.patch = static_cast<unsigned char*>(c->patch_pool[static_cast<size_t>(layer)]);
    a.special = static_cast<unsigned char*>(c->special_pool[static_cast<size_t>(layer)]);
    a.dst = reinterpret_cast<int32_t*>(c->tgt->base) + c0;
    a.n = static_cast<int32_t>(c->blob.size() - c0);
    a.seg_off = static_cast<int32_t>(static_cast<size_t>(c->off_segs) - c0);
    a.nseg = c->n_segs;
    a.max_chunks = c->seg_max_chunks;
    std::memcpy(a.data, c->blob.data() + c0, static_cast<size_t>(a.n) * 4);
    const int e = psw::launch_append_upload(a, hip_stream);
    if (e != 0) return hip_fail(e, "append");
    c->upload_pending = false;
    return PSW_OK;
  }
  if (c->planned && c->n_segs >= 0) {
    psw_status st = flush_plan(c, hip_stream);
    if (st != PSW_OK) return st;
    // segments already in the workspace with the plan
    psw::AppendDevArgs a{};
    a.k = static_cast<const unsigned char*>(k);
    a.v = static_cast<const unsigned char*>(v);
    a.patch = static_cast<unsigned char*>(c->patch_pool[static_cast<size_t>(layer)]);
    a.special = static_cast<unsigned char*>(c->special_pool[static_cast<size_t>(layer)]);
    a.seg = reinterpret_cast<const psw::AppendSeg*>(reinterpret_cast<int32_t*>(c->tgt->base) +
                                                    c->off_segs);
    a.nseg = c->n_segs;
    a.max_chunks = c->seg_max_chunks;
    const int e = psw::launch_append_dev(a, hip_stream);
    if (e != 0) return hip_fail(e, "append");
    return PSW_OK;
  }
  std::vector<psw::AppendSeg> segs;
  for (int32_t b = 0; b < c->cfg.num_streams; ++b) {
    if (c->qo[b + 1] == c->qo[b]) continue;
    psw_status st = frame_segments(c, b, c->qo[b], &segs);
    if (st != PSW_OK) return st;
  }
  return launch_segments(c, layer, k, v, segs, hip_stream);
}

// ---- attention -----------------------------------------------------------------

static void attn_args(psw_cache* c, int32_t layer, const void* q, void* o, float* lse,
                      psw::AttnArgs* out);

// psw_append_attention runs as one launch for the planned frame: the plan
// fits the kernel arguments and the frame's attention is short.  The one
// launch saves the append's launch (a few microseconds) while its tile loop
// runs a few percent slower than the plain kernel's (more scalar registers
// spilled), so frames with more than kFusedMaxScores query-key-head scores
// (the 224x224 frame has 2^26.3, a 1005-row stream over 73128 keys 2^30.1)
// take the two calls.
constexpr int64_t kFusedMaxScores = int64_t{1} << 28;
static bool fusable(const psw_cache* c) {
  const psw_config& cf = c->cfg;
  return c->planned && c->fused_ok && cf.dtype == PSW_BF16 && c->n_items > 0 &&
         c->blob.size() <= static_cast<size_t>(psw::kFusedInts) &&
         c->plan_scores <= kFusedMaxScores;
}


// The plan is made with the list of special pages first; when that list is
// all that keeps a frame from the one-launch form (the plan does not fit the
// kernel arguments but everything else allows the one launch), it is made
// again with the pages as two runs of consecutive ids (when the table has
// them).  Otherwise the list stays: in the 4-wave shape the kernel reading
// the list measured 0.5% faster than the one reading the runs.
psw_status psw_plan(psw_cache* c, void* /*stream*/) {
  PSW_CHECK_CACHE(c);
  if (!c->have_table) return fail(PSW_ESTATE, "no page table built");
  psw_status st = plan_impl(c, false);
  if (st != PSW_OK) return st;
  const bool list_only_obstacle =
      c->fused_ok && c->cfg.dtype == PSW_BF16 && c->n_items > 0 && !c->sids.empty() &&
      c->plan_scores <= kFusedMaxScores && c->blob.size() > static_cast<size_t>(psw::kFusedInts);
  if (!list_only_obstacle) return PSW_OK;
  st = plan_impl(c, true);
  if (st != PSW_OK) return st;
  // without runs the plan just made is the list plan again
  return !c->special_compact || fusable(c) ? PSW_OK : plan_impl(c, false);
}

psw_status psw_plan_fused(psw_cache* c, int32_t* fused) {
  PSW_CHECK_CACHE(c);
  if (fused == nullptr) return fail(PSW_EINVAL, "fused is NULL");
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  *fused = fusable(c) ? 1 : 0;
  return PSW_OK;
}

static psw_status merge_splits(psw_cache* c, const psw::AttnArgs& a, void* o, float* lse,
                               void* hip_stream);

psw_status psw_attention(psw_cache* c, int32_t layer, const void* q, void* o, float* lse,
                         void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  if (c->patch_pool[static_cast<size_t>(layer)] == nullptr)
    return fail(PSW_EUNBOUND, "layer pools not bound");
  if (c->tgt->base == nullptr) return fail(PSW_EUNBOUND, "workspace not bound");
  if (c->n_items > 0 && (q == nullptr || o == nullptr))
    return fail(PSW_EINVAL, "q or o is NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(PSW_EINVAL, "q and o must be 16-byte aligned");
  psw_status fst = flush_plan(c, hip_stream);
  if (fst != PSW_OK) return fst;
  const psw_config& cf = c->cfg;
  psw::AttnArgs a{};
  attn_args(c, layer, q, o, lse, &a);
  int e = 0;
  auto* tm = a.n_items > 0 ? timer_slot(c, &c->t_attn, &e) : nullptr;
  if (e != 0) return hip_fail(e, "attention: timer");
  e = psw::launch_attention(a, cf.dtype == PSW_BF16 ? 0 : 1, c->waves, hip_stream,
                            tm ? tm->first : nullptr, tm ? tm->second : nullptr);
  if (e != 0) return hip_fail(e, "attention");
  return merge_splits(c, a, o, lse, hip_stream);
}

// psw_append_attention on the workspace c->tgt points to.
static psw_status append_attention(psw_cache* c, int32_t layer, const void* k, const void* v,
                                   const void* q, void* o, float* lse, void* hip_stream) {
  const psw_config& cf = c->cfg;
  if (c->tgt->base == nullptr) return fail(PSW_EUNBOUND, "workspace not bound");
  if (!fusable(c)) {
    const psw_status st = psw_append_frames(c, layer, k, v, hip_stream);
    if (st != PSW_OK) return st;
    return psw_attention(c, layer, q, o, lse, hip_stream);
  }
  if (c->patch_pool[static_cast<size_t>(layer)] == nullptr)
    return fail(PSW_EUNBOUND, "layer pools not bound");
  if (k == nullptr || v == nullptr || q == nullptr || o == nullptr)
    return fail(PSW_EINVAL, "k, v, q or o is NULL");
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(o))
    return fail(PSW_EINVAL, "k, v, q and o must be 16-byte aligned");
  psw::FusedArgs f{};
  attn_args(c, layer, q, o, lse, &f.a);
  f.k_in = static_cast<const unsigned char*>(k);
  f.v_in = static_cast<const unsigned char*>(v);
  f.ws_blob = reinterpret_cast<int32_t*>(c->tgt->base);
  f.blob_n = static_cast<int32_t>(c->blob.size());
  f.off_work = c->off_work;
  f.off_pids = c->off_pids;
  f.off_sids = c->off_sids;
  f.off_qo = c->off_qo;
  f.off_segs = c->off_segs;
  f.off_cstart = c->off_cstart;
  f.off_fcur = c->off_fcur;
  f.nseg = c->n_segs;
  f.total_chunks = c->total_chunks;
  f.tokens_per_frame = cf.tokens_per_frame;
  f.num_special = cf.num_special_tokens;
  f.inv_num_special = 1.0f / static_cast<float>(cf.num_special_tokens);
  std::memcpy(f.data, c->blob.data(), c->blob.size() * sizeof(int32_t));
  int e = 0;
  auto* tm = timer_slot(c, &c->t_attn, &e);
  if (e != 0) return hip_fail(e, "attention: timer");
  e = psw::launch_attention_fused(f, c->waves, hip_stream, tm ? tm->first : nullptr,
                                  tm ? tm->second : nullptr);
  if (e != 0) return hip_fail(e, "append + attention");
  c->upload_pending = false;   // the launch wrote the blob to the workspace
  return merge_splits(c, f.a, o, lse, hip_stream);
}

psw_status psw_append_attention(psw_cache* c, int32_t layer, const void* k, const void* v,
                                const void* q, void* o, float* lse, void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  return append_attention(c, layer, k, v, q, o, lse, hip_stream);
}

psw_status psw_append_attention_noalloc(psw_cache* c, int32_t layer, const void* k,
                                        const void* v, const void* q, void* o, float* lse,
                                        void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  // the current plan's layout: ints, then the split records and outputs of
  // its rows only
  const psw_config& cf = c->cfg;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int64_t rows = c->qo[static_cast<size_t>(cf.num_streams)];
  const size_t splits = c->max_split_used > 1 ? static_cast<size_t>(c->max_split_used) : 0;
  WsView view;
  view.part_rows = rows;
  view.ml_off = al(c->blob.size() * sizeof(int32_t));
  view.o_off = view.ml_off + al(splits * rows * cf.num_heads * 4 * sizeof(float));
  const size_t need = view.o_off + al(splits * rows * cf.num_heads * cf.head_dim * 2);
  if (need > psw::kNoAllocScratchBytes)
    return fail(PSW_EINVAL, "plan needs " + std::to_string(need) +
                                " bytes of scratch; the no-alloc entry point holds " +
                                std::to_string(psw::kNoAllocScratchBytes));
  void* base = nullptr;
  const int e = psw::scratch_address(&base);
  if (e != 0) return hip_fail(e, "scratch address");
  view.base = static_cast<unsigned char*>(base);
  // the scratch holds whatever the last call on this GPU left: the plan is
  // written again by this call
  const bool pending = c->upload_pending;
  c->tgt = &view;
  c->upload_pending = true;
  const psw_status st = append_attention(c, layer, k, v, q, o, lse, hip_stream);
  c->tgt = &c->bound;
  c->upload_pending = pending;
  return st;
}

// Attention arguments of the planned frame (pools of `layer`, plan in the
// workspace).
static void attn_args(psw_cache* c, int32_t layer, const void* q, void* o, float* lse,
                      psw::AttnArgs* out) {
  const psw_config& cf = c->cfg;
  int32_t* ints = reinterpret_cast<int32_t*>(c->tgt->base);
  psw::AttnArgs& a = *out;
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.patch_pool = c->patch_pool[static_cast<size_t>(layer)];
  a.special_pool = c->special_pool[static_cast<size_t>(layer)];
  a.work = ints + c->off_work;
  a.patch_ids = ints + c->off_pids;
  a.special_ids = ints + c->off_sids;
  a.special_compact = c->special_compact ? 1 : 0;
  a.part_ml = reinterpret_cast<float*>(c->tgt->base + c->tgt->ml_off);
  a.part_o = reinterpret_cast<uint16_t*>(c->tgt->base + c->tgt->o_off);
  a.n_items = c->n_items;
  a.heads = cf.num_heads;
  a.head_dim = cf.head_dim;
  a.patch_page = c->P;
  a.special_page = cf.special_page_size;
  a.part_rows = static_cast<int32_t>(c->tgt->part_rows);
  a.sm_scale = c->sm_scale;
  a.inv_patch_page = 1.0f / static_cast<float>(c->P);
  a.inv_special_page = 1.0f / static_cast<float>(cf.special_page_size);
  psw::div_magic(static_cast<uint32_t>(c->P), &a.patch_magic, &a.patch_shift);
  psw::div_magic(static_cast<uint32_t>(cf.special_page_size), &a.special_magic,
                 &a.special_shift);
}

// The merge of the split partials, when the plan split any stream.
static psw_status merge_splits(psw_cache* c, const psw::AttnArgs& a, void* o, float* lse,
                               void* hip_stream) {
  const psw_config& cf = c->cfg;
  int32_t* ints = reinterpret_cast<int32_t*>(c->tgt->base);
  int e = 0;
  if (c->max_split_used > 1) {
    psw::MergeArgs m{};
    m.o = o;
    m.lse = lse;
    m.part_o = a.part_o;
    m.part_ml = a.part_ml;
    m.qo_indptr = ints + c->off_qo;
    m.splits = ints + c->off_splits;
    m.num_streams = cf.num_streams;
    m.total_rows = c->qo[static_cast<size_t>(cf.num_streams)];
    m.heads = cf.num_heads;
    m.head_dim = cf.head_dim;
    m.part_rows = a.part_rows;
    m.dtype = cf.dtype == PSW_BF16 ? 0 : 1;
    m.max_splits = c->max_split_used;
    auto* tmm = m.total_rows > 0 ? timer_slot(c, &c->t_merge, &e) : nullptr;
    if (e != 0) return hip_fail(e, "merge: timer");
    e = psw::launch_merge(m, hip_stream, tmm ? tmm->first : nullptr,
                          tmm ? tmm->second : nullptr);
    if (e != 0) return hip_fail(e, "merge");
  }
  return PSW_OK;
}

psw_status psw_visible_tokens(psw_cache* c, int64_t* kv_indptr) {
  PSW_CHECK_CACHE(c);
  if (kv_indptr == nullptr) return fail(PSW_EINVAL, "kv_indptr is NULL");
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  std::copy(c->kv_indptr.begin(), c->kv_indptr.end(), kv_indptr);
  return PSW_OK;
}

// Table fields of the dense check path (pools of `layer`, or none if < 0).
static void dense_args(psw_cache* c, int32_t layer, psw::DenseArgs* d) {
  const psw_config& cf = c->cfg;
  int32_t* ints = reinterpret_cast<int32_t*>(c->tgt->base);
  psw::AttnArgs& a = d->t;
  if (layer >= 0) {
    a.patch_pool = c->patch_pool[static_cast<size_t>(layer)];
    a.special_pool = c->special_pool[static_cast<size_t>(layer)];
  }
  a.work = ints + c->off_work;
  a.patch_ids = ints + c->off_pids;
  a.special_ids = ints + c->off_sids;
  a.special_compact = c->special_compact ? 1 : 0;
  a.n_items = c->n_items;
  a.heads = cf.num_heads;
  a.head_dim = cf.head_dim;
  a.patch_page = c->P;
  a.special_page = cf.special_page_size;
  a.sm_scale = c->sm_scale;
  a.inv_patch_page = 1.0f / static_cast<float>(c->P);
  a.inv_special_page = 1.0f / static_cast<float>(cf.special_page_size);
  d->dtype = cf.dtype == PSW_BF16 ? 0 : 1;
}

psw_status psw_gather_visible_f32(psw_cache* c, int32_t layer, float* k_dense, float* v_dense,
                                  void* hip_stream) {
  PSW_CHECK_CACHE(c);
  PSW_CHECK_LAYER(c, layer);
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  if (c->patch_pool[static_cast<size_t>(layer)] == nullptr)
    return fail(PSW_EUNBOUND, "layer pools not bound");
  if (c->tgt->base == nullptr) return fail(PSW_EUNBOUND, "workspace not bound");
  const bool any = c->kv_indptr.back() > 0;
  if (any && (k_dense == nullptr || v_dense == nullptr))
    return fail(PSW_EINVAL, "k_dense or v_dense is NULL");
  if (!aligned16(k_dense) || !aligned16(v_dense))
    return fail(PSW_EINVAL, "k_dense and v_dense must be 16-byte aligned");
  psw_status fst = flush_plan(c, hip_stream);
  if (fst != PSW_OK) return fst;
  psw::DenseArgs d{};
  dense_args(c, layer, &d);
  d.k_dense = k_dense;
  d.v_dense = v_dense;
  const int e = psw::launch_gather_visible(d, hip_stream);
  if (e != 0) return hip_fail(e, "gather_visible");
  return PSW_OK;
}

psw_status psw_dense_attention_f32(psw_cache* c, const void* q, const float* k_dense,
                                   const float* v_dense, float* o, float* lse,
                                   void* hip_stream) {
  PSW_CHECK_CACHE(c);
  if (!c->planned) return fail(PSW_ESTATE, "no plan: call psw_plan after building the table");
  if (c->tgt->base == nullptr) return fail(PSW_EUNBOUND, "workspace not bound");
  if (c->n_items > 0 &&
      (q == nullptr || k_dense == nullptr || v_dense == nullptr || o == nullptr))
    return fail(PSW_EINVAL, "q, k_dense, v_dense or o is NULL");
  if (!aligned16(q) || !aligned16(k_dense) || !aligned16(v_dense) || !aligned16(o))
    return fail(PSW_EINVAL, "q, k_dense, v_dense and o must be 16-byte aligned");
  psw_status fst = flush_plan(c, hip_stream);
  if (fst != PSW_OK) return fst;
  psw::DenseArgs d{};
  dense_args(c, -1, &d);
  d.t.q = q;
  d.t.lse = lse;
  d.k_dense = const_cast<float*>(k_dense);
  d.v_dense = const_cast<float*>(v_dense);
  d.o = o;
  const int e = psw::launch_dense_attention(d, hip_stream);
  if (e != 0) return hip_fail(e, "dense_attention");
  return PSW_OK;
}

}  // extern "C"
