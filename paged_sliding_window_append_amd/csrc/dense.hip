// Dense float32 check path: the pages' force_fp32 precision mode, which
// gathers the paged K/V into dense tensors and attends over them in float for
// numerical validation ([p1] "How the Paged KV Cache Attention Mechanism
// Enables Long Sequence Inference in LingBot-Map", §Memory Efficiency
// Analysis, precision modes).  Our own kernels, not a library attention:
//
//  * gather_visible_kernel writes every stream's visible tokens, in the
//    visible order of the table, as float rows [token][H][D] (bf16 widened
//    exactly), one row range per stream;
//  * dense_attn_f32_kernel attends each query row over its stream's dense
//    rows in float, with an exact running max, and writes float o and lse.
//
// Both walk the plan's work items: the items of a stream's first query
// block cover its visible tokens once (split after split), and the items of
// a block's first split name each query block once.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device.h"
#include "paging.h"

namespace psw {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// bf16 -> float is exact: the 16 bits are the float's upper half.
__device__ __forceinline__ f32x4 widen_lo(uint32_t a, uint32_t b) {
  return f32x4{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u),
               __uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u)};
}

// grid = (kGatherParts, n_items); workgroup (g, item) takes the g-th of
// kGatherParts contiguous pieces of the item's token range; its 256 threads
// move 8-element pieces of token rows (consecutive threads, consecutive
// bytes of a row).  Workgroups go to the 8 XCDs round-robin by linear index,
// so the piece index runs fastest: the active items' workgroups spread over
// every XCD whichever items are active.
constexpr int kGatherParts = 256;

__global__ __launch_bounds__(256) void gather_visible_kernel(DenseArgs d) {
  const AttnArgs& a = d.t;
  const int32_t* w = a.work + blockIdx.y * kWorkInts;
  if (w[kWQBlock] != 0) return;   // another block of the stream: same tokens
  const int len = w[kWKvEnd] - w[kWKvBegin];
  const int per = (len + kGatherParts - 1) / kGatherParts;
  const int kv_begin = w[kWKvBegin] + static_cast<int>(blockIdx.x) * per;
  const int kv_end = min(w[kWKvEnd], kv_begin + per);
  if (kv_begin >= kv_end) return;
  const int H = a.heads;
  const int per_tok = H * 8;      // pieces of 8 elements per token row
  const int64_t n = static_cast<int64_t>(kv_end - kv_begin) * per_tok;
  const int64_t HD = static_cast<int64_t>(H) * 64;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int j = kv_begin + static_cast<int>(i / per_tok);
    const int e = static_cast<int>(i % per_tok) * 8;   // element in the row
    int64_t ko, vo;
    bool sp;
    token_offsets(a, w, j, &ko, &vo, &sp);
    const int64_t dst = (static_cast<int64_t>(w[kWDenseOff]) + j) * HD + e;
    f32x4* kd = reinterpret_cast<f32x4*>(d.k_dense + dst);
    f32x4* vd = reinterpret_cast<f32x4*>(d.v_dense + dst);
    if (d.dtype == 0) {
      const uint16_t* pool = static_cast<const uint16_t*>(sp ? a.special_pool : a.patch_pool);
      const u32x4 kr = *reinterpret_cast<const u32x4*>(pool + ko + e);
      const u32x4 vr = *reinterpret_cast<const u32x4*>(pool + vo + e);
      kd[0] = widen_lo(kr[0], kr[1]);
      kd[1] = widen_lo(kr[2], kr[3]);
      vd[0] = widen_lo(vr[0], vr[1]);
      vd[1] = widen_lo(vr[2], vr[3]);
    } else {
      const float* pool = static_cast<const float*>(sp ? a.special_pool : a.patch_pool);
      kd[0] = *reinterpret_cast<const f32x4*>(pool + ko + e);
      kd[1] = *reinterpret_cast<const f32x4*>(pool + ko + e + 4);
      vd[0] = *reinterpret_cast<const f32x4*>(pool + vo + e);
      vd[1] = *reinterpret_cast<const f32x4*>(pool + vo + e + 4);
    }
  }
}

// grid = (kMaxQTilesPerBlock, n_items, H); 4 waves.  Workgroup (c, item, h)
// takes query rows [16c, 16c+16) of the item's block for head h (the chunk
// index runs fastest so that the active workgroups spread over the XCDs).  The
// stream's dense K/V rows pass through LDS in tiles of 64 keys (coalesced
// loads by the whole workgroup).  Lane (r, s) = (lane % 16, lane / 16) of
// wave w owns row r and the keys 16 i + 4 w + s of every tile (i = 0..3): a
// sixteenth of the keys, with its own running max, sum and output, updated
// once per tile; the sixteen parts of a row are combined at the end
// (shuffles within the wave, LDS across waves).
constexpr int kDenseTile = 64;
constexpr int kRowF4 = 17;   // 16 float4 per key row + 1 of padding: the
                             // four keys a wave reads at once hit distinct banks

__global__ __launch_bounds__(256) void dense_attn_f32_kernel(DenseArgs d) {
  const AttnArgs& a = d.t;
  const int32_t* w = a.work + blockIdx.y * kWorkInts;
  if (w[kWSplit] > 0) return;     // a block's first split names it once
  const int q_rows = w[kWQRows];
  const int r0 = static_cast<int>(blockIdx.x) * 16;
  if (r0 >= q_rows) return;
  const int h = blockIdx.z;
  const int H = a.heads;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int part = 4 * wave + (lane >> 4);   // key residue mod 16
  const int row = r0 + r;
  const bool live = row < q_rows;
  const int64_t grow = static_cast<int64_t>(w[kWQRow0]) + (live ? row : 0);
  const int64_t HD = static_cast<int64_t>(H) * 64;
  const int64_t kv0 = static_cast<int64_t>(w[kWDenseOff]);
  const int nkv = w[kWKvLen];
  const float c2 = a.sm_scale * kLog2e;

  float q[64];
  if (d.dtype == 0) {
    const uint32_t* qb = static_cast<const uint32_t*>(a.q) + (grow * H + h) * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t u = qb[i];
      q[2 * i] = __uint_as_float(u << 16);
      q[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
    const float* qb = static_cast<const float*>(a.q) + (grow * H + h) * 64;
#pragma unroll
    for (int i = 0; i < 64; ++i) q[i] = qb[i];
  }
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  float m = -INFINITY;   // running max of the raw scores q.k
  float l = 0.f;

  __shared__ f32x4 ks[kDenseTile][kRowF4];
  __shared__ f32x4 vs[kDenseTile][kRowF4];
  // thread tid moves float4 c = tid % 16 of keys tid / 16 + 16 u (u = 0..3);
  // the next tile's pieces are loaded into registers while this one is used
  f32x4 pk[4], pv[4];
  auto load_tile = [&](int base) {
    const int nt = min(kDenseTile, nkv - base);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = (tid >> 4) + 16 * u;
      pk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      pv[u] = pk[u];
      if (key < nt) {
        const int64_t off = (kv0 + base + key) * HD + h * 64 + (tid & 15) * 4;
        pk[u] = *reinterpret_cast<const f32x4*>(d.k_dense + off);
        pv[u] = *reinterpret_cast<const f32x4*>(d.v_dense + off);
      }
    }
  };
  load_tile(0);
  for (int base = 0; base < nkv; base += kDenseTile) {
    const int nt = min(kDenseTile, nkv - base);
    __syncthreads();   // the previous tile is no longer read
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ks[(tid >> 4) + 16 * u][tid & 15] = pk[u];
      vs[(tid >> 4) + 16 * u][tid & 15] = pv[u];
    }
    __syncthreads();
    if (base + kDenseTile < nkv) load_tile(base + kDenseTile);
    float sc[4];
    float mt = m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = part + 16 * i;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 k4 = ks[key][c];
        s = fmaf(q[4 * c], k4[0], s);
        s = fmaf(q[4 * c + 1], k4[1], s);
        s = fmaf(q[4 * c + 2], k4[2], s);
        s = fmaf(q[4 * c + 3], k4[3], s);
      }
      sc[i] = key < nt ? s : -INFINITY;
      mt = fmaxf(mt, sc[i]);
    }
    if (mt == -INFINITY) continue;   // no key of this lane in the tile yet
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mt) * c2);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sc[i] - mt) * c2);
    l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      f32x4 o4 = {acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
      o4 *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v4 = vs[part + 16 * i][c];
        o4[0] = fmaf(p[i], v4[0], o4[0]);
        o4[1] = fmaf(p[i], v4[1], o4[1]);
        o4[2] = fmaf(p[i], v4[2], o4[2]);
        o4[3] = fmaf(p[i], v4[3], o4[3]);
      }
      acc[4 * c] = o4[0];
      acc[4 * c + 1] = o4[1];
      acc[4 * c + 2] = o4[2];
      acc[4 * c + 3] = o4[3];
    }
    m = mt;
  }
  // combine the four parts of a row inside the wave (lanes r, r+16, r+32,
  // r+48); a part that saw no key has m = -inf and weight 0
#pragma unroll
  for (int x = 16; x < 64; x <<= 1) {
    const float mo = __shfl_xor(m, x);
    const float lo = __shfl_xor(l, x);
    const float mn = fmaxf(m, mo);
    const float ws = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
    const float wo = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mo - mn) * c2);
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = acc[i] * ws + __shfl_xor(acc[i], x) * wo;
    l = l * ws + lo * wo;
    m = mn;
  }
  // then across the four waves: [wave][row][m, l, acc[64]]
  __syncthreads();   // the last tile is no longer read
  float (*part_sh)[16][66] = reinterpret_cast<float (*)[16][66]>(&ks[0][0]);
  if (lane < 16) {
    part_sh[wave][r][0] = m;
    part_sh[wave][r][1] = l;
#pragma unroll
    for (int i = 0; i < 64; ++i) part_sh[wave][r][2 + i] = acc[i];
  }
  __syncthreads();
  // 256 threads: row tid / 16, dimensions 4 (tid % 16) .. +3
  const int orow = tid >> 4;
  const int d0 = (tid & 15) * 4;
  if (r0 + orow >= q_rows) return;
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) M = fmaxf(M, part_sh[v][orow][0]);
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float mv = part_sh[v][orow][0];
    const float wv = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mv - M) * c2);
    L += wv * part_sh[v][orow][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += wv * part_sh[v][orow][2 + d0 + i];
  }
  const int64_t g = static_cast<int64_t>(w[kWQRow0]) + r0 + orow;
  const float inv = 1.f / L;
  *reinterpret_cast<f32x4*>(d.o + (g * H + h) * 64 + d0) = o * inv;
  if (d0 == 0 && a.lse != nullptr) a.lse[g * H + h] = M * a.sm_scale + logf(L);
}

}  // namespace

int launch_gather_visible(const DenseArgs& d, void* stream) {
  if (d.t.n_items == 0) return 0;
  hipLaunchKernelGGL(gather_visible_kernel, dim3(kGatherParts, d.t.n_items), dim3(256), 0,
                     static_cast<hipStream_t>(stream), d);
  return static_cast<int>(hipGetLastError());
}

int launch_dense_attention(const DenseArgs& d, void* stream) {
  if (d.t.n_items == 0) return 0;
  hipLaunchKernelGGL(dense_attn_f32_kernel,
                     dim3(kMaxQTilesPerBlock, d.t.n_items, d.t.heads), dim3(256), 0,
                     static_cast<hipStream_t>(stream), d);
  return static_cast<int>(hipGetLastError());
}

}  // namespace psw
