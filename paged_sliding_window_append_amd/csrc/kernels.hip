// HIP kernels for gfx950 (CDNA4): the append_frame K/V write, the table
// upload, the float32 paged prefill attention (the bf16 MFMA kernel lives in
// attention.hip) and the merge of split-KV partial results.
//
// [p1] "How the Paged KV Cache Attention Mechanism Enables Long Sequence
//      Inference in LingBot-Map", §Appending New Frames, §FlashInfer Kernel
//      Execution, §Memory Efficiency Analysis.
// [p3] "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map",
//      §Visible Page Table Attention, §Custom CUDA Kernel Implementation.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "device.h"
#include "launch.h"
#include "paging.h"

namespace psw {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// append_frame: byte copy of contiguous segments (16-byte vectors).
// grid = (max_chunks, nseg); each workgroup copies one 4 KiB chunk.
__global__ __launch_bounds__(256) void append_copy_kernel(AppendArgs a) {
  const int s = blockIdx.y;
  if (s >= a.nseg) return;
  const AppendSeg seg = a.seg[s];
  const int64_t off = static_cast<int64_t>(blockIdx.x) * kAppendChunk +
                      static_cast<int64_t>(threadIdx.x) * 16;
  if (off >= seg.bytes) return;
  const unsigned char* src = (seg.flags & 1) ? a.v : a.k;
  unsigned char* dst = (seg.flags & 2) ? a.special : a.patch;
  const u32x4 val =
      *reinterpret_cast<const u32x4*>(src + seg.src_off + off);
  *reinterpret_cast<u32x4*>(dst + seg.dst_off + off) = val;
}

__global__ __launch_bounds__(256) void append_copy_dev_kernel(AppendDevArgs a) {
  const int s = blockIdx.y;
  if (s >= a.nseg) return;
  const AppendSeg seg = a.seg[s];
  const int64_t off = static_cast<int64_t>(blockIdx.x) * kAppendChunk +
                      static_cast<int64_t>(threadIdx.x) * 16;
  if (off >= seg.bytes) return;
  const unsigned char* src = (seg.flags & 1) ? a.v : a.k;
  unsigned char* dst = (seg.flags & 2) ? a.special : a.patch;
  *reinterpret_cast<u32x4*>(dst + seg.dst_off + off) =
      *reinterpret_cast<const u32x4*>(src + seg.src_off + off);
}

// One launch for the K/V write of a frame and the end of its plan: the
// segment list and the plan ints both come from the kernel arguments.
static_assert(offsetof(AppendUploadArgs, data) % 8 == 0, "segments need 8-byte alignment");
__global__ __launch_bounds__(256) void append_upload_kernel(AppendUploadArgs a) {
  const int s = blockIdx.y;
  if (s == a.nseg) {
    if (blockIdx.x != 0) return;
    const int i = threadIdx.x * 4;
    if (i + 4 <= a.n) {
      *reinterpret_cast<int4*>(a.dst + i) = *reinterpret_cast<const int4*>(a.data + i);
    } else {
      for (int j = i; j < a.n; ++j) a.dst[j] = a.data[j];
    }
    return;
  }
  const AppendSeg seg = reinterpret_cast<const AppendSeg*>(a.data + a.seg_off)[s];
  const int64_t off = static_cast<int64_t>(blockIdx.x) * kAppendChunk +
                      static_cast<int64_t>(threadIdx.x) * 16;
  if (off >= seg.bytes) return;
  const unsigned char* src = (seg.flags & 1) ? a.v : a.k;
  unsigned char* dst = (seg.flags & 2) ? a.special : a.patch;
  *reinterpret_cast<u32x4*>(dst + seg.dst_off + off) =
      *reinterpret_cast<const u32x4*>(src + seg.src_off + off);
}

// ---------------------------------------------------------------------------
// Table upload: the ints travel in the kernel arguments; every thread moves
// 16 bytes, so the whole block is one round trip to argument memory.
__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  const int i = threadIdx.x * 4;
  if (i + 4 <= a.n) {
    *reinterpret_cast<int4*>(a.dst + i) = *reinterpret_cast<const int4*>(a.data + i);
  } else {
    for (int j = i; j < a.n; ++j) a.dst[j] = a.data[j];
  }
}

// ---------------------------------------------------------------------------
// float32 paged prefill attention (validation dtype, small workloads):
// one thread per query row, online softmax over the visible keys in order.
__global__ __launch_bounds__(64) void attn_f32_d64_kernel(AttnArgs a) {
  const int item = blockIdx.x;
  const int h = blockIdx.y;
  const int32_t* w = a.work + item * kWorkInts;
  const int q_row0 = w[kWQRow0];
  const int q_rows = w[kWQRows];
  const int kv_begin = w[kWKvBegin];
  const int kv_end = w[kWKvEnd];
  const int split = w[kWSplit];
  const int H = a.heads;
  const float* qb = static_cast<const float*>(a.q);
  float* ob = static_cast<float*>(a.o);
  const float c2 = a.sm_scale * kLog2e;

  for (int row = threadIdx.x; row < q_rows; row += blockDim.x) {
    const int64_t grow = q_row0 + row;
    float q[64];
    float acc[64];
#pragma unroll
    for (int d = 0; d < 64; ++d) {
      q[d] = qb[(grow * H + h) * 64 + d];
      acc[d] = 0.f;
    }
    float m = -INFINITY;
    float l = 0.f;
    for (int j = kv_begin; j < kv_end; ++j) {
      int64_t ko, vo;
      bool sp;
      token_offsets(a, w, j, &ko, &vo, &sp);
      const float* pool = static_cast<const float*>(sp ? a.special_pool : a.patch_pool);
      const float* kr = pool + ko + h * 64;
      const float* vr = pool + vo + h * 64;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) s = fmaf(q[d], kr[d], s);
      const float m_new = fmaxf(m, s);
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);
      const float p = __builtin_amdgcn_exp2f((s - m_new) * c2);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < 64; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
      m = m_new;
    }
    if (split < 0) {
      const float inv = 1.f / l;
#pragma unroll
      for (int d = 0; d < 64; ++d) ob[(grow * H + h) * 64 + d] = acc[d] * inv;
      if (a.lse != nullptr) a.lse[grow * H + h] = m * a.sm_scale + __logf(l);
    } else {
      const int64_t prow = static_cast<int64_t>(split) * a.part_rows + grow;
      const float inv = 1.f / l;
      float mx = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) mx = fmaxf(mx, fabsf(acc[d] * inv));
      const float k = mx > 0.f ? inv / mx : 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d)
        a.part_o[(prow * H + h) * 64 + d] =
            __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[d] * k));
      *reinterpret_cast<float4*>(a.part_ml + (prow * H + h) * 4) =
          float4{m * a.sm_scale, l, mx, 0.f};
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of split-KV partials: with w_s = e^{m_s - M} l_s,
//   o = sum_s w_s sc_s Ô_s / sum_s w_s,   lse = M + log sum_s w_s,
// where Ô_s is split s's normalized output scaled by 1/sc_s (fp16).
// A lane owns 8 dimensions (16 bytes) of one (row, head) and the splits
// g, g+SG, ..., g+(R-1)SG of its split group g < SG; the 8*SG lanes of a
// (row, head) sit together, so a wave covers 8/SG pairs of adjacent heads,
// each split's rows of them one contiguous read.  SG*R covers the largest
// split count (launch_merge picks the pair).  A lane issues all R record and slice
// loads at once, first thing: their indices are clamped to the launch's
// largest split count, not to the row's stream's (whose load would have to
// come first), so a split past the stream's count reads a row the buffers
// hold but this plan did not write, and selects (not a product with a zero
// weight, which stale bits could turn into a NaN) leave it out.  M, sum w_s
// and the eight sums then reduce over the split groups.
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

template <int SG>
__device__ __forceinline__ float split_groups_max(float x) {
#pragma unroll
  for (int k = 8; k < 8 * SG; k <<= 1) x = fmaxf(x, __shfl_xor(x, k));
  return x;
}
template <int SG>
__device__ __forceinline__ float split_groups_sum(float x) {
#pragma unroll
  for (int k = 8; k < 8 * SG; k <<= 1) x += __shfl_xor(x, k);
  return x;
}

template <int SG, int R>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  static_assert(SG * R <= kMaxSplits, "split groups");
  const int lane = threadIdx.x & 63;
  const int dc = lane & 7;
  const int sg = (lane >> 3) & (SG - 1);
  const int H = a.heads;
  const int rh = ((blockIdx.x * 4 + (threadIdx.x >> 6)) * 8 + (lane >> 3)) / SG;
  // lanes past the last pair only take part in the shuffles (no barrier here)
  const bool valid = rh < a.total_rows * H;
  const int row = valid ? rh / H : 0;
  const int h = valid ? rh - row * H : 0;
  const int64_t stride = static_cast<int64_t>(a.part_rows) * H;   // per split
  const float4* rec = reinterpret_cast<const float4*>(a.part_ml) +
                      static_cast<int64_t>(row) * H + h;
  const uint16_t* po = a.part_o + (static_cast<int64_t>(row) * H + h) * 64 + 8 * dc;
  float4 r[R];
  u32x4 pv[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int s = min(sg + SG * k, a.max_splits - 1);
    r[k] = rec[s * stride];
    pv[k] = *reinterpret_cast<const u32x4*>(po + s * stride * 64);
  }
  int b = 0;
  while (b + 1 < a.num_streams && row >= a.qo_indptr[b + 1]) ++b;
  const int ns = valid ? a.splits[b] : 0;   // <= 1: the attention kernel wrote the row
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < R; ++k)
    if (sg + SG * k < ns) m = fmaxf(m, r[k].x);
  M = split_groups_max<SG>(m);
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool in = sg + SG * k < ns;
    const float wgt = in ? __builtin_amdgcn_exp2f((r[k].x - M) * kLog2e) * r[k].y : 0.f;
    l += wgt;
    const float ws = in ? wgt * r[k].z : 0.f;
    const f16x8 o = __builtin_bit_cast(f16x8, in ? pv[k] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws, static_cast<float>(o[i]), acc[i]);
  }
  L = split_groups_sum<SG>(l);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = split_groups_sum<SG>(acc[i]);
  if (sg != 0 || ns <= 1) return;
  const float inv = 1.f / L;
  const int64_t oi = (static_cast<int64_t>(row) * H + h) * 64 + 8 * dc;
  if (a.dtype == 0) {
    bf16x8 ob;
#pragma unroll
    for (int i = 0; i < 8; ++i) ob[i] = static_cast<__bf16>(acc[i] * inv);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.o) + oi) = ob;
  } else {
    float* of = static_cast<float*>(a.o) + oi;
    *reinterpret_cast<float4*>(of) = float4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<float4*>(of + 4) =
        float4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (dc == 0 && a.lse != nullptr) a.lse[static_cast<int64_t>(row) * H + h] = M + __logf(L);
}

}  // namespace

// ---------------------------------------------------------------------------
int device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  return static_cast<int>(e);
}

int launch_upload(const UploadArgs& a, void* stream) {
  hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_append(const AppendArgs& a, void* stream) {
  if (a.nseg <= 0) return 0;
  hipLaunchKernelGGL(append_copy_kernel, dim3(a.max_chunks, a.nseg), dim3(256),
                     0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_attention(const AttnArgs& a, int dtype, int waves, void* stream, void* ev0,
                     void* ev1) {
  if (a.n_items <= 0) return 0;
  if (dtype == 0) return launch_attention_bf16(a, waves, stream, ev0, ev1);
  launch_timed(attn_f32_d64_kernel, dim3(a.n_items, a.heads), dim3(64), stream, ev0, ev1, a);
  return static_cast<int>(hipGetLastError());
}

int launch_append_dev(const AppendDevArgs& a, void* stream) {
  if (a.nseg <= 0) return 0;
  hipLaunchKernelGGL(append_copy_dev_kernel, dim3(a.max_chunks, a.nseg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_append_upload(const AppendUploadArgs& a, void* stream) {
  hipLaunchKernelGGL(append_upload_kernel, dim3(a.max_chunks > 0 ? a.max_chunks : 1, a.nseg + 1),
                     dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

int launch_merge(const MergeArgs& a, void* stream, void* ev0, void* ev1) {
  if (a.total_rows <= 0) return 0;
  // split groups SG and splits per lane R covering max_splits: R at most 4
  // (more lanes per row, fewer loads each, so more waves share the wait)
  // up to 32 splits
  const int ms = a.max_splits;
  const int sg = ms <= 4 ? 1 : ms <= 8 ? 2 : ms <= 16 ? 4 : 8;
  const int64_t lanes8 = static_cast<int64_t>(a.total_rows) * a.heads * sg;   // 8-lane groups
  const dim3 grid(static_cast<unsigned>((lanes8 + 31) / 32));   // 32 groups per workgroup
  if (ms <= 2)
    launch_timed(merge_kernel<1, 2>, grid, dim3(256), stream, ev0, ev1, a);
  else if (ms <= 4)
    launch_timed(merge_kernel<1, 4>, grid, dim3(256), stream, ev0, ev1, a);
  else if (ms <= 8)
    launch_timed(merge_kernel<2, 4>, grid, dim3(256), stream, ev0, ev1, a);
  else if (ms <= 16)
    launch_timed(merge_kernel<4, 4>, grid, dim3(256), stream, ev0, ev1, a);
  else if (ms <= 32)
    launch_timed(merge_kernel<8, 4>, grid, dim3(256), stream, ev0, ev1, a);
  else
    launch_timed(merge_kernel<8, 8>, grid, dim3(256), stream, ev0, ev1, a);
  return static_cast<int>(hipGetLastError());
}

const char* hip_error_text(int err) {
  return hipGetErrorString(static_cast<hipError_t>(err));
}

int timer_create(void** ev) {
  hipEvent_t e = nullptr;
  const hipError_t r = hipEventCreate(&e);
  *ev = e;
  return static_cast<int>(r);
}

int timer_elapsed_ms(void* start, void* stop, float* ms) {
  hipError_t r = hipEventSynchronize(static_cast<hipEvent_t>(stop));
  if (r != hipSuccess) return static_cast<int>(r);
  return static_cast<int>(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start),
                                              static_cast<hipEvent_t>(stop)));
}

int timer_destroy(void* ev) {
  return static_cast<int>(hipEventDestroy(static_cast<hipEvent_t>(ev)));
}

}  // namespace psw
