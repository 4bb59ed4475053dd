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
#pragma unroll
      for (int d = 0; d < 64; ++d) a.part_o[(prow * H + h) * 64 + d] = acc[d];
      a.part_ml[(prow * H + h) * 2] = m * a.sm_scale;
      a.part_ml[(prow * H + h) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of split-KV partials: o = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s
// One wave per (row, head): lane s holds split s's (m, l) (at most 64
// splits), lane d accumulates output dimension d.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rh >= a.total_rows * a.heads) return;
  const int H = a.heads;
  const int row = rh / H;
  const int h = rh - row * H;
  int b = 0;
  while (b + 1 < a.num_streams && row >= a.qo_indptr[b + 1]) ++b;
  const int ns = a.splits[b];
  if (ns <= 1) return;
  float m = -INFINITY;
  float l = 0.f;
  if (lane < ns) {
    const int64_t prow = static_cast<int64_t>(lane) * a.part_rows + row;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (prow * H + h) * 2);
    m = ml.x;
    l = ml.y;
  }
  const float M = wave_max(m);
  const float wgt = lane < ns ? __builtin_amdgcn_exp2f((m - M) * kLog2e) : 0.f;
  const float L = wave_sum(wgt * l);
  const float* po = a.part_o + (static_cast<int64_t>(row) * H + h) * 64 + lane;
  const int64_t split_stride = static_cast<int64_t>(a.part_rows) * H * 64;
  float acc = 0.f;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    const float o0 = po[(s + 0) * split_stride];
    const float o1 = po[(s + 1) * split_stride];
    const float o2 = po[(s + 2) * split_stride];
    const float o3 = po[(s + 3) * split_stride];
    acc += __shfl(wgt, s) * o0 + __shfl(wgt, s + 1) * o1 + __shfl(wgt, s + 2) * o2 +
           __shfl(wgt, s + 3) * o3;
  }
  for (; s < ns; ++s) acc += __shfl(wgt, s) * po[s * split_stride];
  const float val = acc / L;
  const int64_t oi = (static_cast<int64_t>(row) * H + h) * 64 + lane;
  if (a.dtype == 0)
    static_cast<__bf16*>(a.o)[oi] = static_cast<__bf16>(val);
  else
    static_cast<float*>(a.o)[oi] = val;
  if (lane == 0 && a.lse != nullptr) a.lse[static_cast<int64_t>(row) * H + h] = M + __logf(L);
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

int launch_attention(const AttnArgs& a, int dtype, void* stream, void* ev0, void* ev1) {
  if (a.n_items <= 0) return 0;
  if (dtype == 0) return launch_attention_bf16(a, stream, ev0, ev1);
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
  launch_timed(merge_kernel, dim3((a.total_rows * a.heads + 3) / 4), dim3(256), stream, ev0,
               ev1, a);
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
