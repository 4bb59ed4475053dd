// HIP kernels for gfx950 (CDNA4): the append_frame K/V write, the table
// upload, the paged prefill attention (bf16 on MFMA, plus a plain float32
// variant) and the merge of split-KV partial results.
//
// [p1] "How the Paged KV Cache Attention Mechanism Enables Long Sequence
//      Inference in LingBot-Map", §Appending New Frames, §FlashInfer Kernel
//      Execution, §Memory Efficiency Analysis.
// [p3] "FlashInfer Paged KV Cache Performance Benefits in LingBot-Map",
//      §Visible Page Table Attention, §Custom CUDA Kernel Implementation.
//
// The attention reads K/V straight from the pages listed in the visible
// table (no dense gather), stages each 64-key tile in LDS once per
// workgroup and shares it between all query rows of the frame, computes
// S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16, and keeps
// the softmax state (running max and sum) in float registers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.h"

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

// ---------------------------------------------------------------------------
// Table upload: the ints travel in the kernel arguments.
__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) a.dst[i] = a.data[i];
}

// ---------------------------------------------------------------------------
// Visible token j of a stream -> element offset of its K row (head 0) in
// the patch or special pool; the V row follows at +page_size*H*D.
template <typename T>
__device__ __forceinline__ void token_rows(const AttnArgs& a,
                                           const int32_t* w, int j,
                                           const T** krow, const T** vrow) {
  const int64_t HD = static_cast<int64_t>(a.heads) * a.head_dim;
  const int patch_tok = w[kWPatchTok];
  if (j < patch_tok) {
    const int pi = j / a.patch_page;
    const int slot = j - pi * a.patch_page;
    const int64_t page = a.patch_ids[w[kWPatchOff] + pi];
    const T* base = static_cast<const T*>(a.patch_pool) +
                    (page * 2 * a.patch_page + slot) * HD;
    *krow = base;
    *vrow = base + static_cast<int64_t>(a.patch_page) * HD;
  } else {
    const int s = j - patch_tok;
    const int pi = s / a.special_page;
    const int slot = s - pi * a.special_page;
    const int64_t page = a.special_ids[w[kWSpecialOff] + pi];
    const T* base = static_cast<const T*>(a.special_pool) +
                    (page * 2 * a.special_page + slot) * HD;
    *krow = base;
    *vrow = base + static_cast<int64_t>(a.special_page) * HD;
  }
}

// ---------------------------------------------------------------------------
// bf16 paged prefill attention, head_dim 64.
//
// Workgroup = one work item x one head, 4 waves.  Query tile qt (16 rows)
// belongs to wave qt % 4, register slot qt / 4.  KV tiles of 64 keys are
// staged in LDS: K row-major [key][d], V transposed [d][key].
//
// MFMA 16x16x32 bf16 lane layout used below (l = lane, g = l / 16,
// r = l % 16): A operand rows are r with k-slots g*8..g*8+7, B operand
// columns are r with the same k-slots, and C element i of lane l is row
// g*4+i, column r.  Scores are computed transposed, S^T = K Q^T, so a lane
// holds 16 keys of a single query and the row max and sum need only two
// cross-lane steps.  The K rows fed to the A operand are permuted so that
// lane group g ends up with keys 32c + 8g + 0..7 (c = 0, 1): exactly the
// k-slots the B operand of O^T += V^T P^T needs, so P never moves between
// lanes.
constexpr int kLdsStride = 72;   // bf16 per LDS row: 64 + 8 padding

template <int NQT>
__global__ __launch_bounds__(256) void attn_bf16_d64_kernel(AttnArgs a) {
  const int item = blockIdx.x;
  const int h = blockIdx.y;
  const int32_t* w = a.work + item * kWorkInts;
  const int q_row0 = w[kWQRow0];
  const int q_rows = w[kWQRows];
  const int kv_begin = w[kWKvBegin];
  const int kv_end = w[kWKvEnd];
  const int split = w[kWSplit];

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKvTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][64 * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int H = a.heads;
  const float c2 = a.sm_scale * kLog2e;

  const int nqt = (q_rows + kQTileRows - 1) / kQTileRows;
  // number of this wave's valid register slots
  const int my_tiles = nqt > wave ? (nqt - wave + kWaves - 1) / kWaves : 0;

  // ---- Q^T fragments (B operand of S^T = K Q^T), held for the whole run
  bf16x8 qf[NQT][2];
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = (wave + t * kWaves) * kQTileRows + r16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < my_tiles && row < q_rows)
        v = *reinterpret_cast<const u32x4*>(
            qbase + (static_cast<int64_t>(q_row0 + row) * H + h) * 64 +
            kk * 32 + g * 8);
      qf[t][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[NQT][4];
  float m_run[NQT];
  float l_run[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: thread handles tile rows (tid>>3) and (tid>>3)+32, chunk
  // tid&7 (8 bf16 = 16 bytes) of K and of V.
  const int st_row = tid >> 3;
  const int st_chunk = tid & 7;
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int j = kv_begin + tile * kKvTile + st_row + rr * 32;
      kreg[rr] = u32x4{0u, 0u, 0u, 0u};
      vreg[rr] = u32x4{0u, 0u, 0u, 0u};
      if (j < kv_end) {
        const uint16_t* kr;
        const uint16_t* vr;
        token_rows<uint16_t>(a, w, j, &kr, &vr);
        kreg[rr] = *reinterpret_cast<const u32x4*>(kr + h * 64 + st_chunk * 8);
        vreg[rr] = *reinterpret_cast<const u32x4*>(vr + h * 64 + st_chunk * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = st_row + rr * 32;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * kLdsStride + st_chunk * 8]) =
          kreg[rr];
      const uint32_t words[4] = {vreg[rr][0], vreg[rr][1], vreg[rr][2],
                                 vreg[rr][3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t val =
            static_cast<uint16_t>(words[e >> 1] >> ((e & 1) * 16));
        Vt[buf][(st_chunk * 8 + e) * kLdsStride + row] = val;
      }
    }
  };

  const int ntiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) load_tile(tile + 1);

    if (my_tiles > 0) {
      // ---- S^T = K Q^T for 4 blocks of 16 keys
      f32x4 s[NQT][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = 32 * (kb >> 1) + (r16 >> 2) * 8 + (kb & 1) * 4 + (r16 & 3);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 kf = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(
                          &Ks[buf][key * kLdsStride + kk * 32 + g * 8]));
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            if (t < my_tiles) {
              const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
              s[t][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  kf, qf[t][kk], kk == 0 ? zero : s[t][kb], 0, 0, 0);
            }
          }
        }
      }

      // ---- mask keys past the end (last tile only)
      const int valid = kv_end - (kv_begin + tile * kKvTile);
      if (valid < kKvTile) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 32 * (kb >> 1) + g * 8 + (kb & 1) * 4 + i;
            if (key >= valid) {
#pragma unroll
              for (int t = 0; t < NQT; ++t) s[t][kb][i] = -INFINITY;
            }
          }
        }
      }

      // ---- online softmax, P packed to bf16
      bf16x8 pf[NQT][2];
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        if (t < my_tiles) {
          float mx = s[t][0][0];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kb][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float m_new = fmaxf(m_run[t], mx);
          const float alpha = __builtin_amdgcn_exp2f((m_run[t] - m_new) * c2);
          m_run[t] = m_new;
          const float mc = m_new * c2;
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(s[t][kb][i], c2, -mc));
              s[t][kb][i] = p;
              rs += p;
            }
          l_run[t] = l_run[t] * alpha + rs;
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[t][db] *= alpha;
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pf[t][cc][i] = static_cast<__bf16>(s[t][2 * cc][i]);
              pf[t][cc][4 + i] = static_cast<__bf16>(s[t][2 * cc + 1][i]);
            }
          }
        }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(
                          &Vt[buf][(db * 16 + r16) * kLdsStride + cc * 32 + g * 8]));
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            if (t < my_tiles)
              oacc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  vf, pf[t][cc], oacc[t][db], 0, 0, 0);
          }
        }
      }
    }

    if (tile + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  uint16_t* obase = static_cast<uint16_t*>(a.o);
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    if (t >= my_tiles) continue;
    float l = l_run[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int row = (wave + t * kWaves) * kQTileRows + r16;
    if (row >= q_rows) continue;
    const int64_t grow = q_row0 + row;
    if (split < 0) {
      const float inv = 1.f / l;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint32_t packed[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const __bf16 lo = static_cast<__bf16>(oacc[t][db][2 * i] * inv);
          const __bf16 hi = static_cast<__bf16>(oacc[t][db][2 * i + 1] * inv);
          packed[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        uint2 pv;
        pv.x = packed[0];
        pv.y = packed[1];
        *reinterpret_cast<uint2*>(obase + (grow * H + h) * 64 + db * 16 + g * 4) = pv;
      }
      if (g == 0 && a.lse != nullptr)
        a.lse[grow * H + h] = m_run[t] * a.sm_scale + __logf(l);
    } else {
      const int64_t prow = static_cast<int64_t>(split) * a.part_rows + grow;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *reinterpret_cast<f32x4*>(a.part_o + (prow * H + h) * 64 + db * 16 + g * 4) =
            oacc[t][db];
      if (g == 0) {
        float2 ml;
        ml.x = m_run[t] * a.sm_scale;
        ml.y = l;
        *reinterpret_cast<float2*>(a.part_ml + (prow * H + h) * 2) = ml;
      }
    }
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
      const float* kr;
      const float* vr;
      token_rows<float>(a, w, j, &kr, &vr);
      kr += h * 64;
      vr += h * 64;
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
// grid = (rows, ceil(H / 4)), block = 256 (4 heads x 64 dims).
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  if (h >= a.heads || d >= a.head_dim) return;
  int b = 0;
  while (b + 1 < a.num_streams && row >= a.qo_indptr[b + 1]) ++b;
  const int ns = a.splits[b];
  if (ns <= 1) return;
  const int H = a.heads;
  const int D = a.head_dim;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    const int64_t prow = static_cast<int64_t>(s) * a.part_rows + row;
    M = fmaxf(M, a.part_ml[(prow * H + h) * 2]);
  }
  float L = 0.f;
  float acc = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t prow = static_cast<int64_t>(s) * a.part_rows + row;
    const float wgt = __builtin_amdgcn_exp2f((a.part_ml[(prow * H + h) * 2] - M) * kLog2e);
    L += wgt * a.part_ml[(prow * H + h) * 2 + 1];
    acc += wgt * a.part_o[(prow * H + h) * D + d];
  }
  const float val = acc / L;
  const int64_t oi = (static_cast<int64_t>(row) * H + h) * D + d;
  if (a.dtype == 0)
    static_cast<__bf16*>(a.o)[oi] = static_cast<__bf16>(val);
  else
    static_cast<float*>(a.o)[oi] = val;
  if (d == 0 && a.lse != nullptr) a.lse[static_cast<int64_t>(row) * H + h] = M + __logf(L);
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

int launch_attention(const AttnArgs& a, int dtype, void* stream) {
  if (a.n_items <= 0) return 0;
  const dim3 grid(a.n_items, a.heads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == 0)
    hipLaunchKernelGGL(attn_bf16_d64_kernel<kMaxQTilesPerWave>, grid,
                       dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_f32_d64_kernel, grid, dim3(64), 0, s, a);
  return static_cast<int>(hipGetLastError());
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.total_rows <= 0) return 0;
  const dim3 grid(a.total_rows, (a.heads + 3) / 4);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
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

int timer_record(void* ev, void* stream) {
  return static_cast<int>(hipEventRecord(static_cast<hipEvent_t>(ev),
                                         static_cast<hipStream_t>(stream)));
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
