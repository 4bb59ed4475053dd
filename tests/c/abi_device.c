/* A plain C99 caller of libpsw.so on the GPU: device memory from the HIP
 * runtime's C API, every step of the frame through the C ABI, no Python and
 * no torch.  Reads a workload and its inputs from a file, streams the frames
 * (begin, evict, visible table, plan, then append + attention in one call
 * per frame) and writes each frame's o and lse to another file, for the
 * test that compares them with the oracle.
 *
 *   abi_device <inputs.bin> <outputs.bin>
 *
 * inputs.bin: 12 int32 (magic 0x70737731, frames, streams, T, Ns, Ps, S, W,
 * H, D, max_patch_pages, max_special_pages), then per frame q, k and v as
 * bf16 bit patterns [streams*T][H][D], stream after stream.  outputs.bin:
 * per frame o (bf16 bits, [streams*T][H][D]) then lse (float32,
 * [streams*T][H]).  Exit status 0 on success; a message on stderr else. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "psw.h"

#define CHECK_PSW(x)                                                        \
  do {                                                                      \
    psw_status st_ = (x);                                                   \
    if (st_ != PSW_OK) {                                                    \
      fprintf(stderr, "%s: %d %s\n", #x, (int)st_, psw_last_error());       \
      return 1;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 1;                                                             \
    }                                                                       \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: abi_device <inputs.bin> <outputs.bin>\n");
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  FILE* out = fopen(argv[2], "wb");
  if (in == NULL || out == NULL) {
    fprintf(stderr, "cannot open the files\n");
    return 1;
  }
  int32_t hd[12];
  if (fread(hd, sizeof(int32_t), 12, in) != 12 || hd[0] != 0x70737731) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const int frames = hd[1], B = hd[2], T = hd[3];
  psw_config cfg = {0};
  cfg.num_layers = 1;
  cfg.num_streams = B;
  cfg.tokens_per_frame = T;
  cfg.num_special_tokens = hd[4];
  cfg.special_page_size = hd[5];
  cfg.scale_frames = hd[6];
  cfg.sliding_window = hd[7];
  cfg.num_heads = hd[8];
  cfg.head_dim = hd[9];
  cfg.max_patch_pages = hd[10];
  cfg.max_special_pages = hd[11];
  cfg.dtype = PSW_BF16;
  cfg.include_scale_frames = 1;
  cfg.cross_frame_special = 1;
  CHECK_PSW(psw_config_check(&cfg));

  size_t patch_bytes = 0, special_bytes = 0, ws_bytes = 0;
  CHECK_PSW(psw_pool_bytes(&cfg, &patch_bytes, &special_bytes, &ws_bytes));
  const size_t rows = (size_t)B * (size_t)T;
  const size_t frame_elems = rows * (size_t)cfg.num_heads * (size_t)cfg.head_dim;
  void *patch = NULL, *special = NULL, *ws = NULL, *q = NULL, *k = NULL, *v = NULL, *o = NULL;
  float* lse = NULL;
  CHECK_HIP(hipMalloc(&patch, patch_bytes));
  CHECK_HIP(hipMalloc(&special, special_bytes));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc(&q, frame_elems * 2));
  CHECK_HIP(hipMalloc(&k, frame_elems * 2));
  CHECK_HIP(hipMalloc(&v, frame_elems * 2));
  CHECK_HIP(hipMalloc(&o, frame_elems * 2));
  CHECK_HIP(hipMalloc((void**)&lse, rows * (size_t)cfg.num_heads * sizeof(float)));
  uint16_t* host_in = (uint16_t*)malloc(3 * frame_elems * 2);
  uint16_t* host_o = (uint16_t*)malloc(frame_elems * 2);
  float* host_lse = (float*)malloc(rows * (size_t)cfg.num_heads * sizeof(float));
  if (host_in == NULL || host_o == NULL || host_lse == NULL) {
    fprintf(stderr, "out of host memory\n");
    return 1;
  }

  psw_cache* c = NULL;
  CHECK_PSW(psw_create(&cfg, &c));
  CHECK_PSW(psw_bind_layer(c, 0, patch, special));
  CHECK_PSW(psw_bind_workspace(c, ws, ws_bytes));
  for (int t = 0; t < frames; ++t) {
    if (fread(host_in, 2, 3 * frame_elems, in) != 3 * frame_elems) {
      fprintf(stderr, "short input at frame %d\n", t);
      return 1;
    }
    for (int b = 0; b < B; ++b) {
      CHECK_PSW(psw_begin_frame(c, b));
      CHECK_PSW(psw_evict_frames(c, b));
    }
    CHECK_PSW(psw_build_visible_page_table(c));
    CHECK_PSW(psw_plan(c, NULL));
    CHECK_HIP(hipMemcpy(q, host_in, frame_elems * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(k, host_in + frame_elems, frame_elems * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, host_in + 2 * frame_elems, frame_elems * 2, hipMemcpyHostToDevice));
    CHECK_PSW(psw_append_attention(c, 0, k, v, q, o, lse, NULL));
    CHECK_HIP(hipMemcpy(host_o, o, frame_elems * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(host_lse, lse, rows * (size_t)cfg.num_heads * sizeof(float),
                        hipMemcpyDeviceToHost));
    fwrite(host_o, 2, frame_elems, out);
    fwrite(host_lse, sizeof(float), rows * (size_t)cfg.num_heads, out);
  }
  psw_destroy(c);
  CHECK_HIP(hipFree(patch));
  CHECK_HIP(hipFree(special));
  CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipFree(q));
  CHECK_HIP(hipFree(k));
  CHECK_HIP(hipFree(v));
  CHECK_HIP(hipFree(o));
  CHECK_HIP(hipFree(lse));
  free(host_in);
  free(host_o);
  free(host_lse);
  fclose(in);
  fclose(out);
  return 0;
}
