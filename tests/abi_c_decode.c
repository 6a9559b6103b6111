/* One decode step from a plain C99 caller: inputs read from raw files,
 * device buffers from hipMalloc, the three calls of the step on the null
 * stream, outputs written back to files -- no C++ or torch anywhere in the
 * process.  Used by tests/test_gpu_abi_c.py, which writes the inputs and
 * checks the outputs.
 *
 * usage: abi_c_decode DIR   (DIR holds meta.txt and the .bin inputs) */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

static const char* g_dir;

static void* read_file(const char* name, size_t* bytes) {
  char path[4096];
  FILE* f;
  long n;
  void* buf;
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  fseek(f, 0, SEEK_END);
  n = ftell(f);
  fseek(f, 0, SEEK_SET);
  buf = malloc(n > 0 ? (size_t)n : 1);
  if (!buf || fread(buf, 1, (size_t)n, f) != (size_t)n) {
    fprintf(stderr, "cannot read %s\n", path);
    exit(2);
  }
  fclose(f);
  *bytes = (size_t)n;
  return buf;
}

static void write_file(const char* name, const void* buf, size_t bytes) {
  char path[4096];
  FILE* f;
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

#define HIP_OK(x)                                                   \
  do {                                                              \
    hipError_t e_ = (x);                                            \
    if (e_ != hipSuccess) {                                         \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));       \
      exit(3);                                                      \
    }                                                               \
  } while (0)

#define MLA_OK_(x)                                                  \
  do {                                                              \
    int s_ = (x);                                                   \
    if (s_ != MLA_OK) {                                             \
      fprintf(stderr, "%s: %s\n", #x, mla_status_string(s_));       \
      exit(4);                                                      \
    }                                                               \
  } while (0)

/* host file -> new device buffer */
static void* upload(const char* name, size_t* bytes) {
  void* d = NULL;
  void* h = read_file(name, bytes);
  HIP_OK(hipMalloc(&d, *bytes ? *bytes : 1));
  HIP_OK(hipMemcpy(d, h, *bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

int main(int argc, char** argv) {
  mla_dims_t dims;
  long long row_width, mbps, max_seq_len, causal, paged;
  double softmax_scale, rope_base;
  size_t n;
  FILE* f;
  char meta[4096];
  void *q_nope, *q_rope, *positions, *w_uk, *w_uv, *rows, *seq_lens, *block_table = NULL;
  void *q_abs, *o_part, *lse_part, *o, *lse;
  int64_t ob, lb, rows_q, q_abs_bytes, o_bytes, lse_bytes;
  int32_t G;
  void* host;

  if (argc != 2) return 1;
  g_dir = argv[1];
  snprintf(meta, sizeof meta, "%s/meta.txt", g_dir);
  f = fopen(meta, "r");
  if (!f) return 2;
  memset(&dims, 0, sizeof dims);
  if (fscanf(f, "%d %d %d %d %d %d %d %d %d %lld %lld %lld %lld %lld %lf %lf", &dims.batch,
             &dims.q_len, &dims.heads, &dims.d_nope, &dims.d_rope, &dims.d_latent, &dims.d_v,
             &dims.q_dtype, &dims.kv_dtype, &row_width, &mbps, &max_seq_len, &causal, &paged,
             &softmax_scale, &rope_base) != 16)
    return 2;
  fclose(f);

  q_nope = upload("q_nope.bin", &n);
  q_rope = upload("q_rope.bin", &n);
  positions = upload("positions.bin", &n);
  w_uk = upload("w_uk.bin", &n);
  w_uv = upload("w_uv.bin", &n);
  rows = upload("rows.bin", &n);
  seq_lens = upload("seq_lens.bin", &n);
  if (paged) block_table = upload("block_table.bin", &n);

  /* caller-owned buffers, sized from the library's own helpers */
  MLA_OK_(mla_num_splits_hint(&dims, 0, &G));
  MLA_OK_(mla_workspace_bytes(&dims, G, &ob, &lb));
  rows_q = (int64_t)dims.batch * dims.q_len * dims.heads;
  q_abs_bytes = rows_q * (dims.d_latent + dims.d_rope) * 2; /* fp16 for bf16 queries */
  o_bytes = rows_q * dims.d_v * 2;
  lse_bytes = rows_q * 4;
  HIP_OK(hipMalloc(&q_abs, (size_t)q_abs_bytes));
  HIP_OK(hipMalloc(&o_part, (size_t)ob));
  HIP_OK(hipMalloc(&lse_part, (size_t)lb));
  HIP_OK(hipMalloc(&o, (size_t)o_bytes));
  HIP_OK(hipMalloc(&lse, (size_t)lse_bytes));

  MLA_OK_(mla_absorb_q(&dims, q_nope, q_rope, (const int32_t*)positions, (float)rope_base, w_uk,
                       q_abs, NULL));
  MLA_OK_(mla_decode_attn(&dims, q_abs, rows, (const char*)rows + (size_t)dims.d_latent * 2,
                          row_width, NULL, (const int32_t*)seq_lens, (const int32_t*)block_table,
                          (int32_t)mbps, 64, (int32_t)max_seq_len, (int32_t)causal,
                          (float)softmax_scale, G, o_part, (float*)lse_part, NULL));
  MLA_OK_(mla_combine_out_proj(&dims, G, (const int32_t*)seq_lens, o_part, (const float*)lse_part,
                               w_uv, o, (float*)lse, NULL, NULL));
  HIP_OK(hipDeviceSynchronize());

  host = malloc((size_t)o_bytes);
  HIP_OK(hipMemcpy(host, o, (size_t)o_bytes, hipMemcpyDeviceToHost));
  write_file("o.bin", host, (size_t)o_bytes);
  free(host);
  host = malloc((size_t)lse_bytes);
  HIP_OK(hipMemcpy(host, lse, (size_t)lse_bytes, hipMemcpyDeviceToHost));
  write_file("lse.bin", host, (size_t)lse_bytes);
  free(host);
  printf("num_splits %d\n", G);
  return 0;
}
