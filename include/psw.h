/*
 * psw.h -- paged sliding-window two-stream KV cache and paged prefill
 * attention for AMD MI355X (gfx950).  C ABI.
 *
 * Pages cited (by title; sections named at each call):
 *   [p1] "How the Paged KV Cache Attention Mechanism Enables Long Sequence
 *        Inference in LingBot-Map"
 *   [p2] "KV Cache Mechanism in LingBot-Map for Streaming Inference: A Deep
 *        Dive"
 *   [p3] "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map:
 *        Technical Implementation and Benchmarks"
 *   [p4] "How LingBot-Map Achieves ~20 FPS Inference with Its KV Cache"
 *
 * Model of the cache.  Each of B video streams owns, per layer, a patch
 * stream (one page per frame, recyclable: permanent scale pages plus a
 * sliding window, evicted pages back on a free list) and a special stream
 * (append-only pages holding every frame's special tokens, never evicted)
 * ([p1] §Two-Stream Page Design; [p2] §Two-Stream Design).  One frame step:
 *
 *   for each stream b:  psw_begin_frame(b); psw_evict_frames(b);
 *   psw_build_visible_page_table();  psw_plan(stream);        -- once/frame
 *   for each layer l:   psw_append_frames(l, k, v); psw_attention(l, q, o)
 *                       (or psw_append_attention(l, k, v, q, o): the same
 *                       in one launch when the plan fits its arguments)
 *
 * ([p1] §Runtime Flow for Frame Processing; [p3] §Visible Page Table
 * Attention: the table is built once per frame and every layer reuses it.)
 *
 * Conventions.
 *  - Ownership: the caller owns every device buffer (pools, q/k/v/o/lse and
 *    the workspace) and keeps them alive while the cache uses them.  The
 *    library owns only host bookkeeping and never allocates device memory;
 *    its one device buffer is the static scratch array that
 *    psw_append_attention_noalloc uses in place of a workspace.
 *  - Streams: `hip_stream` is a hipStream_t (NULL = the null stream).  All
 *    device work of a call is enqueued on it; no call waits for the device.
 *    Calls on one cache that touch the device must be ordered by the caller
 *    (simplest: one stream per cache).
 *  - Errors: every call returns a psw_status.  A failing call changes no
 *    state (strong guarantee); psw_last_error() gives a thread-local message.
 *  - Layout ([p1] §Physical Memory Layout, read as one pool per page
 *    stream, with the axis of size 2 holding K (0) and V (1)):
 *        patch pool   [B * max_patch_pages][2][P ][H][D]
 *        special pool [B * max_special_pages][2][Ps][H][D]
 *    with P = tokens_per_frame - num_special_tokens.  Stream b owns patch
 *    pages [b*max_patch_pages, (b+1)*max_patch_pages) and special pages
 *    [b*max_special_pages, (b+1)*max_special_pages).  q, k, v and o are
 *    [rows][H][D], lse is [rows][H] float; rows of a frame: special tokens
 *    first ([0, Ns)), then patches ([Ns, T)).
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef PSW_H
#define PSW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PSW_OK = 0,
  PSW_EINVAL = -1,          /* bad argument or configuration */
  PSW_ENOPAGE = -2,         /* patch free list empty */
  PSW_ESPECIAL_FULL = -3,   /* special pool cannot take another frame */
  PSW_ESTATE = -4,          /* call not valid in the current state */
  PSW_EHIP = -5,            /* a HIP runtime call failed */
  PSW_EUNBOUND = -6         /* pools or workspace not bound */
} psw_status;

typedef enum { PSW_BF16 = 0, PSW_FP32 = 1 } psw_dtype;

/* Constructor arguments ([p1] §Implementation Example; [p2] §Configuration
 * Parameters).  The eviction parameters are fixed here; the pages pass them
 * again on every eviction call, always with the same values. */
typedef struct {
  int32_t num_layers;          /* one pool pair per layer ("block") */
  int32_t num_streams;         /* B independent videos, batched */
  int32_t num_heads;           /* H query heads = H KV heads */
  int32_t head_dim;            /* D; 64 */
  int32_t dtype;               /* psw_dtype of q/k/v/o and the pools */
  int32_t tokens_per_frame;    /* T (patches + specials) */
  int32_t num_special_tokens;  /* Ns >= 1 */
  int32_t special_page_size;   /* Ps >= 1 */
  int32_t scale_frames;        /* S >= 0: first kept frames, permanent */
  int32_t sliding_window;      /* W >= 0: recent frames kept */
  int32_t include_scale_frames; /* 1: keep S scale frames; 0: none (S acts as 0) */
  int32_t cross_frame_special; /* 1: specials of evicted frames stay visible;
                                  0: only those of frames whose patch pages
                                  are visible ([p2] §Configuration Parameters) */
  int32_t max_patch_pages;     /* per stream, >= S + W + 1 */
  int32_t max_special_pages;   /* per stream, >= 1 */
  int32_t max_kv_splits;       /* 0 -> 64; at most 64; bounds the workspace */
  float sm_scale;              /* 0 -> 1/sqrt(D) */
  int32_t max_frames_per_step; /* 0 -> 1; at most 64: frames one stream may
                                  begin at once (psw_begin_frames); bounds
                                  the workspace */
} psw_config;

/* get_cache_stats record ([p3] §Monitoring Cache Statistics). */
typedef struct {
  int32_t frame_count;     /* frames kept (evicted ones included) */
  int32_t scale_pages;
  int32_t live_pages;      /* window pages resident */
  int32_t free_pages;
  int32_t special_tokens;
} psw_stats;

/* Visible page table in CSR form over the B streams ([p1] §Building the
 * Visible Page Table; [p1] FAQ on variable token counts).  A stream without
 * a current frame has empty ranges.  Visible tokens of stream b, in order:
 * every listed patch page whole (P tokens), then the visible special tokens:
 * the first special_head_len[b] tokens of the listed special pages (from
 * slot 0 of the first), then special_tail_len[b] tokens starting at slot
 * special_tail_first[b] of the page that follows the head's
 * ceil(head_len / Ps) pages.  With cross-frame specials the head is every
 * special token written so far and the tail is empty; without, the head is
 * the scale frames' tokens and the tail the visible window frames'.
 * special_last_len[b] is the fill of the last listed page (1..Ps).  Host
 * pointers.  In psw_set_page_table the three head/tail arrays may be NULL:
 * then every token of the listed pages is visible (the head); qo lengths
 * must be k*T with 0 <= k <= max_frames_per_step. */
typedef struct {
  int32_t num_streams;
  const int32_t* qo_indptr;          /* [B+1] query rows (T per frame) */
  const int32_t* patch_indptr;       /* [B+1] */
  const int32_t* patch_ids;          /* global patch page IDs, table order */
  const int32_t* special_indptr;     /* [B+1] */
  const int32_t* special_ids;        /* global special page IDs */
  const int32_t* special_last_len;   /* [B] */
  const int32_t* special_head_len;   /* [B] */
  const int32_t* special_tail_first; /* [B] */
  const int32_t* special_tail_len;   /* [B] */
} psw_page_table;

typedef struct psw_cache psw_cache;

/* Thread-local text of the last error ("" if none). */
const char* psw_last_error(void);

/* Checks a configuration without creating anything.  Besides the ranges
 * above, each of 2*B*max_patch_pages*P (K and V rows of the patch pool),
 * 2*B*max_special_pages*Ps (of the special pool) and B*64*T (rows of one
 * step's k/v input at the most frames per step) must be below 2^29: the
 * attention kernel keeps a row index and two flags in one 32-bit word.
 * PSW_EINVAL otherwise. */
psw_status psw_config_check(const psw_config* cfg);

/* Bytes of one layer's patch pool and special pool, and of the device
 * workspace (page table, plan and split-KV partials). */
psw_status psw_pool_bytes(const psw_config* cfg, size_t* patch_pool_bytes,
                          size_t* special_pool_bytes, size_t* workspace_bytes);

/* Creates the host bookkeeping of every stream: all patch pages free, no
 * frames ([p1] §Implementation Example, constructor). */
psw_status psw_create(const psw_config* cfg, psw_cache** out);
void psw_destroy(psw_cache* cache);

/* Binds layer `layer`'s pools (device, caller-owned, sizes from
 * psw_pool_bytes).  Their contents need no initialisation. */
psw_status psw_bind_layer(psw_cache* cache, int32_t layer, void* patch_pool,
                          void* special_pool);

/* Binds the device workspace (caller-owned, >= workspace_bytes). */
psw_status psw_bind_workspace(psw_cache* cache, void* workspace, size_t bytes);

/* Empties stream `stream` (-1: every stream) for a new video: the cache
 * reset between videos ([p2] §Manual Cache Control). */
psw_status psw_reset(psw_cache* cache, int32_t stream);

/* Bookkeeping half of append_frame ([p1] §Appending New Frames; [p2]
 * §Patch Stream): takes the top page of the free stack for the new frame
 * (a scale page while fewer than S are held, else a window page) and
 * reserves the next Ns special slots.  The frame becomes the stream's
 * current frame.  ENOPAGE / ESPECIAL_FULL when a pool is exhausted. */
psw_status psw_begin_frame(psw_cache* cache, int32_t stream);

/* Joint prefill of n consecutive frames ([p2] §Sliding-Window Eviction
 * Strategy and the FAQ on disabling the window: the scale frames keep a
 * bidirectional context, read as the first S frames prefilled together).
 * The same as n begin_frame calls in a row, except that the n frames form
 * the stream's current chunk: the table gives the stream n*T query rows
 * (frame after frame, each [specials, patches]), every one of them attends
 * over the visible set that holds all n frames, and the append writes the
 * n frames' K/V ([n*T][H][D]) to their pages and special slots.  A rollback
 * undoes the whole chunk.  EINVAL if n is outside [1, max_frames_per_step]
 * or, for n > 1, more than W of the n frames would become window pages (an
 * eviction would then take a page of the chunk). */
psw_status psw_begin_frames(psw_cache* cache, int32_t stream, int32_t n);

/* Sliding-window eviction ([p1] §Evicting Stale Frames; [p2]
 * §Sliding-Window Eviction Strategy): while more than W window pages are
 * resident, the oldest goes back on the free stack.  Scale and special
 * pages are never touched.  While eviction is deferred it is only recorded.
 * An eviction that removes a page ends the current frame's undo window. */
psw_status psw_evict_frames(psw_cache* cache, int32_t stream);

/* Deferred eviction and rollback ([p2] §Flow-Based Keyframe Selection; [p4]
 * §Deferred Eviction and Rollback Mechanism). */
psw_status psw_set_defer_eviction(psw_cache* cache, int32_t stream, int32_t on);
/* Commit: runs the eviction now, whatever the defer flag says. */
psw_status psw_execute_deferred_eviction(psw_cache* cache, int32_t stream);
/* Undoes the last begin_frame exactly: its page back on top of the free
 * stack, its special slots released, frame count restored.  ESTATE if there
 * is no such frame (never begun, already rolled back, or an eviction removed
 * a page since).  The stream then has no current frame. */
psw_status psw_rollback_last_frame(psw_cache* cache, int32_t stream);

/* K/V write of append_frame ([p1] §Appending New Frames): k, v are one
 * frame [T][H][D] on the device (a chunk of n frames: [n*T][H][D], frame
 * after frame); rows [0, Ns) go to the stream's special slots, rows [Ns, T)
 * to its current patch page.  ESTATE if the stream has no current frame. */
psw_status psw_append_frame(psw_cache* cache, int32_t layer, int32_t stream,
                            const void* k, const void* v, void* hip_stream);

/* Same for every stream of the last built table at once: k, v are
 * [qo_indptr[B]][H][D], stream after stream, as the table's qo_indptr (T
 * rows per current frame, n*T per current chunk). */
psw_status psw_append_frames(psw_cache* cache, int32_t layer, const void* k,
                             const void* v, void* hip_stream);

/* Builds the visible page table on the host from the bookkeeping: for
 * each stream with a current frame, the scale pages, the most recent W
 * window pages, all special pages written so far and the fill of the last
 * one ([p1] §Building the Visible Page Table).  No device work. */
psw_status psw_build_visible_page_table(psw_cache* cache);

/* Host view of the last built (or set) table; valid until the next build. */
psw_status psw_get_page_table(psw_cache* cache, psw_page_table* out);

/* Replaces the current table by a caller's one (copied).  Page IDs must be
 * in the streams' ranges and qo lengths k*T (0 <= k <= max_frames_per_step). */
psw_status psw_set_page_table(psw_cache* cache, const psw_page_table* table);

/* Plan ([p3] §Visible Page Table Attention, plan once per frame): splits
 * the attention work over workgroups for the current table and stages table
 * and plan on the host (no workspace needed for this call).  They reach the workspace with the next
 * psw_append_frames or psw_attention call, on that call's stream (the
 * append of the frame carries the last 3840 bytes in its own launch), so a
 * frame costs no separate upload launch.  hip_stream is not used (kept for
 * the plan/run call shape); calls after the first that read the plan on
 * another stream must be ordered after it by the caller. */
psw_status psw_plan(psw_cache* cache, void* hip_stream);

/* Run ([p1] §FlashInfer Kernel Execution; [p3] §Custom CUDA Kernel
 * Implementation): paged prefill attention of layer `layer` over the
 * planned table.  For each stream b, head h and query row i of its frame:
 *   o[i,h]   = sum_j softmax_j(q[i,h].k[j,h] * sm_scale) v[j,h]
 *   lse[i,h] = ln sum_j exp(q[i,h].k[j,h] * sm_scale)
 * over the stream's visible tokens j, with no mask among them.  q, o:
 * [qo_indptr[B]][H][D] (dtype); lse: [qo_indptr[B]][H] float (may be NULL).
 * bf16 runs on MFMA with float accumulation and a float softmax. */
psw_status psw_attention(psw_cache* cache, int32_t layer, const void* q,
                         void* o, float* lse, void* hip_stream);

/* psw_append_frames followed by psw_attention on the same layer, with the
 * same arguments and the same results ([p1] §Runtime Flow for Frame
 * Processing: a block appends its frame's K/V, then attends).
 *
 * One kernel launch (plus the split merge) when all of these hold: bf16; a
 * table built by psw_build_visible_page_table; a plan of at most 944 ints
 * (the 262-token frame of one stream fits; when the listed special pages
 * alone push it past that, psw_plan gives each stream's special pages as
 * its two runs of consecutive ids, head and tail, which such a table always
 * has, so a long video's growing list does not count); at most 2^28 query x
 * visible token x head scores (where saving a launch outweighs the one-launch
 * kernel's slightly slower tile loop).  The workgroups then also write the
 * frames' K/V into the pools and read those frames' rows straight from k
 * and v.  Otherwise it makes the two calls.
 *
 * k, v: [qo_indptr[B]][H][D] like q, device memory, caller-owned; they must
 * stay unchanged until the launch has run.  Errors as the two calls
 * (ESTATE without a plan, EINVAL for a bad layer or NULL/misaligned
 * pointers, EUNBOUND without pools). */
psw_status psw_append_attention(psw_cache* cache, int32_t layer, const void* k,
                                const void* v, const void* q, void* o, float* lse,
                                void* hip_stream);

/* psw_append_attention for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same calls, kernels and results, with one difference: the
 * device workspace (the plan, and the split-KV records and outputs) is the
 * library's own scratch array of PSW_NOALLOC_SCRATCH_BYTES (32 MiB) instead
 * of the bound workspace, so no workspace need be bound.  The caller still
 * passes and owns q, k, v, o, lse and the bound pools.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); the scratch
 * is a static device array that each GPU the library runs on holds until the
 * process ends.  Its first call on a device looks up that device's copy.
 *
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other caches, other threads) race, so the caller must
 * order them.  Each call writes the plan and every split record and output
 * it reads before reading it, so whatever an earlier call left in the
 * scratch does not matter.
 *
 * Errors as psw_append_attention, plus EINVAL when the plan needs more than
 * PSW_NOALLOC_SCRATCH_BYTES (256-byte aligned: the plan ints, then
 * splits * rows * H * 16 bytes of records and splits * rows * H * D * 2
 * bytes of outputs, with splits = the plan's largest KV split count when it
 * splits and rows = qo_indptr[B]) and EHIP when the scratch cannot be
 * found on the current device. */
#define PSW_NOALLOC_SCRATCH_BYTES (32u << 20)
psw_status psw_append_attention_noalloc(psw_cache* cache, int32_t layer, const void* k,
                                        const void* v, const void* q, void* o, float* lse,
                                        void* hip_stream);

/* *fused = 1 when psw_append_attention runs the planned frame as one launch,
 * 0 when it makes the two calls.  ESTATE without a plan. */
psw_status psw_plan_fused(psw_cache* cache, int32_t* fused);

/* Dense float32 check path, the pages' force_fp32 precision mode ([p1]
 * §Memory Efficiency Analysis: the paged K/V gathered into dense tensors and
 * attended in float, for numerical validation).  Own kernels, no library
 * attention.  Each call needs a plan (psw_plan) and uses its table.
 *
 * psw_visible_tokens: fills the host array kv_indptr [B+1]: stream b's
 * visible tokens are the dense rows [kv_indptr[b], kv_indptr[b+1]).
 *
 * psw_gather_visible_f32: writes layer `layer`'s visible K and V of every
 * stream as float rows k_dense, v_dense [kv_indptr[B]][H][D] (device,
 * caller-owned), in the table's visible order (listed patch pages whole,
 * then the special head and tail); bf16 values are widened exactly.
 *
 * psw_dense_attention_f32: for each stream b, head h and query row i of its
 * frame, attention over b's dense rows in float with an exact running max:
 * o (float [qo_indptr[B]][H][D]) and lse (float [qo_indptr[B]][H], may be
 * NULL), with the definitions of psw_attention; q in the cache dtype.  The
 * dense rows may come from psw_gather_visible_f32 or from the caller. */
psw_status psw_visible_tokens(psw_cache* cache, int64_t* kv_indptr);
psw_status psw_gather_visible_f32(psw_cache* cache, int32_t layer, float* k_dense,
                                  float* v_dense, void* hip_stream);
psw_status psw_dense_attention_f32(psw_cache* cache, const void* q, const float* k_dense,
                                   const float* v_dense, float* o, float* lse,
                                   void* hip_stream);

/* Statistics of one stream ([p3] §Monitoring Cache Statistics). */
psw_status psw_get_cache_stats(psw_cache* cache, int32_t stream,
                               psw_stats* out);

/* Free stack of one stream, bottom first, as global page IDs; *n is the
 * count (call with cap 0 to size the buffer). */
psw_status psw_export_free_list(psw_cache* cache, int32_t stream, int32_t* buf,
                                int32_t cap, int32_t* n);

/* Kernel timing (diagnostics, for roofline figures).  While enabled, every
 * attention-kernel and merge-kernel launch carries a pair of HIP events that
 * the runtime stamps at the start and the end of that kernel's dispatch on
 * its stream (hipExtLaunchKernelGGL), so no extra packets enter the stream
 * and the kernels' own durations are unchanged; each stamped launch still
 * delays the next launch by a few microseconds, so a caller that also times
 * the stream should enable it for a sample of launches only.
 * psw_profile_read waits for the recorded events, returns the summed
 * durations in milliseconds and the launch counts, and clears them. */
psw_status psw_profile_enable(psw_cache* cache, int32_t on);
psw_status psw_profile_read(psw_cache* cache, double* attention_ms,
                            int32_t* attention_launches, double* merge_ms,
                            int32_t* merge_launches);

/* Number of workgroups and KV splits of the current plan (diagnostics). */
psw_status psw_plan_info(psw_cache* cache, int32_t* work_items,
                         int32_t* max_splits_used);

/* Waves per workgroup of the current plan's attention launch: 4 (two
 * workgroups per compute unit) or 8 (one per compute unit, half the KV
 * splits), the plan's choice by the frame's size (diagnostics).
 * PSW_ESTATE without a plan. */
psw_status psw_plan_waves(psw_cache* cache, int32_t* waves);

#ifdef __cplusplus
}
#endif

#endif /* PSW_H */
