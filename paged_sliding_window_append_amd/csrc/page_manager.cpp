// Host bookkeeping of one video stream (see page_manager.h for the pages'
// sections this follows).
//
// Readings where the pages say nothing: the free list is a LIFO stack whose
// first pops are pages 0, 1, 2, ...; scale pages are the first kept frames;
// eviction runs before attention so the window count includes the current
// frame; a rollback is the exact inverse of the last begin (one frame or a
// chunk), so it is refused once an eviction has removed a page after that
// begin.  A chunk of n frames is n single-frame allocations in a row.
#include "page_manager.h"

#include <algorithm>

namespace psw {

Err StreamBook::init(const StreamConfig& cfg) {
  if (cfg.scale_frames < 0 || cfg.sliding_window < 0 || cfg.num_special < 1 ||
      cfg.special_page < 1 || cfg.max_special_pages < 1 ||
      cfg.max_patch_pages < cfg.scale_frames + cfg.sliding_window + 1)
    return Err::inval;
  cfg_ = cfg;
  reset();
  return Err::ok;
}

void StreamBook::reset() {
  free_.clear();
  free_.reserve(static_cast<size_t>(cfg_.max_patch_pages));
  for (int32_t p = cfg_.max_patch_pages - 1; p >= 0; --p) free_.push_back(p);
  scale_.clear();
  scale_.reserve(static_cast<size_t>(cfg_.scale_frames));
  window_.init(cfg_.max_patch_pages);
  n_special_ = 0;
  frame_count_ = 0;
  defer_ = false;
  pending_ = false;
  undo_n_ = 0;
  undo_scale_n_ = 0;
  cur_pages_.clear();
  cur_special_ = 0;
}

Err StreamBook::begin_frames(int32_t n) {
  if (n < 1) return Err::inval;
  const int32_t to_scale =
      std::min(n, cfg_.scale_frames - static_cast<int32_t>(scale_.size()));
  if (n > 1 && n - to_scale > cfg_.sliding_window) return Err::inval;
  if (static_cast<int32_t>(free_.size()) < n) return Err::nopage;
  const int64_t cap =
      static_cast<int64_t>(cfg_.max_special_pages) * cfg_.special_page;
  if (static_cast<int64_t>(n_special_) + static_cast<int64_t>(n) * cfg_.num_special > cap)
    return Err::special_full;
  cur_pages_.clear();
  for (int32_t f = 0; f < n; ++f) {
    const int32_t page = free_.back();
    free_.pop_back();
    if (f < to_scale)
      scale_.push_back(page);
    else
      window_.push_back(page);
    cur_pages_.push_back(page);
  }
  undo_n_ = n;
  undo_scale_n_ = to_scale;
  cur_special_ = n_special_;
  n_special_ += n * cfg_.num_special;
  frame_count_ += n;
  return Err::ok;
}

int32_t StreamBook::evict_now() {
  int32_t n = 0;
  while (window_.size() > cfg_.sliding_window) {
    free_.push_back(window_.pop_front());
    ++n;
  }
  pending_ = false;
  if (n > 0) undo_n_ = 0;
  return n;
}

Err StreamBook::evict(int32_t* evicted) {
  int32_t n = 0;
  if (defer_)
    pending_ = window_.size() > cfg_.sliding_window;
  else
    n = evict_now();
  if (evicted) *evicted = n;
  return Err::ok;
}

Err StreamBook::execute_deferred_eviction(int32_t* evicted) {
  const int32_t n = evict_now();
  if (evicted) *evicted = n;
  return Err::ok;
}

Err StreamBook::rollback_last_frame() {
  if (undo_n_ == 0) return Err::state;
  for (int32_t f = undo_n_ - 1; f >= 0; --f) {
    if (f < undo_scale_n_)
      scale_.pop_back();
    else
      window_.pop_back();
    free_.push_back(cur_pages_[static_cast<size_t>(f)]);   // last popped goes back first
  }
  n_special_ -= undo_n_ * cfg_.num_special;
  frame_count_ -= undo_n_;
  pending_ = false;
  undo_n_ = 0;
  undo_scale_n_ = 0;
  cur_pages_.clear();
  cur_special_ = 0;
  return Err::ok;
}

void StreamBook::visible_patch_pages(std::vector<int32_t>* out,
                                     int32_t base) const {
  for (int32_t p : scale_) out->push_back(base + p);
  const int32_t n = window_.size();
  const int32_t start = n > cfg_.sliding_window ? n - cfg_.sliding_window : 0;
  for (int32_t i = start; i < n; ++i) out->push_back(base + window_.at(i));
}

void StreamBook::visible_special_segments(int32_t* head_len, int32_t* tail_start,
                                          int32_t* tail_end) const {
  const int32_t n = n_special_;
  *tail_start = *tail_end = 0;
  if (cfg_.cross_frame_special || n == 0) {
    *head_len = n;
    return;
  }
  const int32_t head = static_cast<int32_t>(scale_.size()) * cfg_.num_special;
  const int32_t vis_window = std::min(cfg_.sliding_window, window_.size());
  const int32_t tail = (frame_count_ - vis_window) * cfg_.num_special;   // >= head
  if (tail == head) {
    *head_len = n;
    return;
  }
  *head_len = head;
  if (tail < n) {
    *tail_start = tail;
    *tail_end = n;
  }
}

int32_t StreamBook::special_pages(int32_t* last_len) const {
  if (n_special_ == 0) {
    *last_len = 0;
    return 0;
  }
  const int32_t np = (n_special_ + cfg_.special_page - 1) / cfg_.special_page;
  *last_len = n_special_ - (np - 1) * cfg_.special_page;
  return np;
}

}  // namespace psw
