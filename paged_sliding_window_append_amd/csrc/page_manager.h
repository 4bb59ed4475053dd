// Host bookkeeping of one video stream: patch pages (free stack, scale
// pages, sliding window) and the append-only special stream.
//
// [p1] "How the Paged KV Cache Attention Mechanism Enables Long Sequence
//      Inference in LingBot-Map", §Two-Stream Page Design, §Runtime Flow.
// [p2] "KV Cache Mechanism in LingBot-Map for Streaming Inference: A Deep
//      Dive", §Patch Stream (Recyclable), §Sliding-Window Eviction Strategy,
//      §Flow-Based Keyframe Selection.
// [p3] "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map",
//      §Monitoring Cache Statistics.
// [p4] "How LingBot-Map Achieves ~20 FPS Inference with Its KV Cache",
//      §Deferred Eviction and Rollback Mechanism.
//
// Everything is O(1) per frame except the table build, which is linear in
// the visible pages.  Page IDs here are local to the stream.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace psw {

enum class Err : int {
  ok = 0,
  inval = -1,
  nopage = -2,
  special_full = -3,
  state = -4,
};

struct StreamConfig {
  int32_t scale_frames;     // S
  int32_t sliding_window;   // W
  int32_t num_special;      // Ns
  int32_t special_page;     // Ps
  int32_t max_patch_pages;  // pool pages of this stream
  int32_t max_special_pages;
  int32_t cross_frame_special;  // 0: only visible frames' specials are visible
};

// A ring of page IDs with O(1) push at the back and pop at both ends.  The
// window never holds more than max_patch_pages entries.
class PageRing {
 public:
  void init(int32_t capacity) {
    buf_.assign(static_cast<size_t>(capacity > 0 ? capacity : 1), 0);
    head_ = 0;
    size_ = 0;
  }
  int32_t size() const { return size_; }
  int32_t at(int32_t i) const {  // 0 = oldest
    return buf_[static_cast<size_t>((head_ + i) % cap())];
  }
  int32_t back() const { return at(size_ - 1); }
  void push_back(int32_t v) {
    buf_[static_cast<size_t>((head_ + size_) % cap())] = v;
    ++size_;
  }
  int32_t pop_front() {
    int32_t v = buf_[static_cast<size_t>(head_)];
    head_ = (head_ + 1) % cap();
    --size_;
    return v;
  }
  int32_t pop_back() {
    --size_;
    return buf_[static_cast<size_t>((head_ + size_) % cap())];
  }

 private:
  int32_t cap() const { return static_cast<int32_t>(buf_.size()); }
  std::vector<int32_t> buf_;
  int32_t head_ = 0;
  int32_t size_ = 0;
};

class StreamBook {
 public:
  Err init(const StreamConfig& cfg);
  void reset();

  // Allocation for a new frame: top of the free stack becomes a scale page
  // while fewer than S are held, else the newest window page; the next Ns
  // special slots are reserved.  Strong guarantee on failure.
  Err begin_frame() { return begin_frames(1); }
  // The same for n consecutive frames at once, which then form the current
  // chunk (joint prefill of several frames, e.g. the S scale frames: their
  // queries attend together over a table that holds all of them).  For
  // n > 1 at most W of them may become window pages, so no eviction can
  // take a page of the chunk.  Strong guarantee on failure.
  Err begin_frames(int32_t n);
  // Pops window pages while more than W are resident (recorded only while
  // eviction is deferred).  Returns the number evicted through *evicted.
  Err evict(int32_t* evicted);
  void set_defer(bool on) { defer_ = on; }
  Err execute_deferred_eviction(int32_t* evicted);
  Err rollback_last_frame();

  bool has_current() const { return !cur_pages_.empty(); }
  // frames of the current chunk (1 after begin_frame) and their pages
  int32_t current_frames() const { return static_cast<int32_t>(cur_pages_.size()); }
  int32_t current_page(int32_t f) const { return cur_pages_[static_cast<size_t>(f)]; }
  // special position of the chunk's first token (frame f: + f * Ns)
  int32_t current_special_start() const { return cur_special_; }

  // Visible patch pages: scale pages, then the last W window pages.
  void visible_patch_pages(std::vector<int32_t>* out, int32_t base) const;
  // Number of special pages written so far and the fill of the last one.
  int32_t special_pages(int32_t* last_len) const;
  // Visible special-token positions: [0, *head_len) and [*tail_start,
  // *tail_end) (empty when equal).  Kept frame f owns positions
  // [f*Ns, (f+1)*Ns): with cross-frame specials the head is every position
  // written; without, the head is the scale frames' and the tail the last
  // visible window frames'.
  void visible_special_segments(int32_t* head_len, int32_t* tail_start,
                                int32_t* tail_end) const;

  int32_t frame_count() const { return frame_count_; }
  int32_t scale_pages() const { return static_cast<int32_t>(scale_.size()); }
  int32_t live_pages() const { return window_.size(); }
  int32_t free_pages() const { return static_cast<int32_t>(free_.size()); }
  int32_t special_tokens() const { return n_special_; }
  bool deferred() const { return defer_; }
  bool pending() const { return pending_; }
  const std::vector<int32_t>& free_stack() const { return free_; }

 private:
  int32_t evict_now();

  StreamConfig cfg_{};
  std::vector<int32_t> free_;   // stack, top = back()
  std::vector<int32_t> scale_;
  PageRing window_;             // oldest first
  int32_t n_special_ = 0;
  int32_t frame_count_ = 0;
  bool defer_ = false;
  bool pending_ = false;
  // Undo record of the last begin: its frame count (0: nothing to undo) and
  // how many of them went to the scale list (the first ones); the pages are
  // cur_pages_.
  int32_t undo_n_ = 0;
  int32_t undo_scale_n_ = 0;
  // Current chunk: pages of its frames, in frame order, where the per-layer
  // K/V writes go (empty: no current frame), and its first special position.
  std::vector<int32_t> cur_pages_;
  int32_t cur_special_ = 0;
};

}  // namespace psw
