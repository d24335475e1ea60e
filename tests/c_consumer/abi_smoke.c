/*
 * A plain C consumer of the library: one table build and one decode step
 * through include/lsh_attn.h, with device memory from the HIP runtime API and
 * no Python or PyTorch in the process.
 *
 * usage: abi_smoke <dir>
 *   <dir>/meta.txt     B Hq Hkv N d K L T stride scale (text)
 *   <dir>/keys.bin, values.bin   [B,Hkv,N,d] bf16
 *   <dir>/W.bin        [d, L*K] bf16
 *   <dir>/q.bin        [B,Hq,d] bf16
 * writes <dir>/out.bin [B,Hq,d] f32, lse.bin [B,Hq] f32, nsel.bin [B,Hq] i32,
 *        offsets.bin, indices.bin (uint16, the build's outputs)
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lsh_attn.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

#define HIP_OK(x)                                                         \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
      return 1;                                                           \
    }                                                                     \
  } while (0)

#define LSH_OK_(x)                                                        \
  do {                                                                    \
    lsh_status s_ = (x);                                                  \
    if (s_ != LSH_OK) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, lsh_status_string(s_));     \
      return 1;                                                           \
    }                                                                     \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  int B, Hq, Hkv, N, d, K, L, T, stride;
  float scale;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d %f", &B, &Hq, &Hkv, &N, &d, &K, &L, &T, &stride, &scale) != 10) {
      fprintf(stderr, "cannot read %s\n", path);
      return 2;
    }
    fclose(f);
  }
  const size_t kv_bytes = (size_t)B * Hkv * N * d * 2, w_bytes = (size_t)d * L * K * 2, q_bytes = (size_t)B * Hq * d * 2;
  const int nch = lsh_num_chunks(N, stride);
  const size_t off_bytes = (size_t)B * Hkv * L * nch * ((size_t)1 << K) * 2, idx_bytes = (size_t)B * Hkv * L * N * 2;
  void* h_keys = read_file(dir, "keys.bin", kv_bytes);
  void* h_vals = read_file(dir, "values.bin", kv_bytes);
  void* h_w = read_file(dir, "W.bin", w_bytes);
  void* h_q = read_file(dir, "q.bin", q_bytes);
  if (!h_keys || !h_vals || !h_w || !h_q) {
    fprintf(stderr, "missing or short input file in %s\n", dir);
    return 2;
  }

  void *keys, *vals, *w, *q, *bws, *dws;
  uint16_t *offsets, *indices;
  float *out, *lse;
  int32_t* nsel;
  const size_t bws_bytes = lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, LSH_BF16);
  const size_t dws_bytes = lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride);
  if (!bws_bytes || !dws_bytes) {
    fprintf(stderr, "unsupported sizes\n");
    return 2;
  }
  HIP_OK(hipMalloc(&keys, kv_bytes));
  HIP_OK(hipMalloc(&vals, kv_bytes));
  HIP_OK(hipMalloc(&w, w_bytes));
  HIP_OK(hipMalloc(&q, q_bytes));
  HIP_OK(hipMalloc((void**)&offsets, off_bytes));
  HIP_OK(hipMalloc((void**)&indices, idx_bytes));
  HIP_OK(hipMalloc(&bws, bws_bytes));
  HIP_OK(hipMalloc(&dws, dws_bytes));
  HIP_OK(hipMalloc((void**)&out, (size_t)B * Hq * d * sizeof(float)));
  HIP_OK(hipMalloc((void**)&lse, (size_t)B * Hq * sizeof(float)));
  HIP_OK(hipMalloc((void**)&nsel, (size_t)B * Hq * sizeof(int32_t)));
  HIP_OK(hipMemcpy(keys, h_keys, kv_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(vals, h_vals, kv_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, h_w, w_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(q, h_q, q_bytes, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  LSH_OK_(lsh_build_tables(keys, w, B, Hkv, N, d, K, L, stride, LSH_BF16, offsets, indices, NULL, bws, bws_bytes,
                           (void*)stream));
  LSH_OK_(lsh_decode_attention(q, keys, vals, w, indices, offsets, B, Hq, Hkv, N, d, K, L, T, stride, scale,
                               LSH_BF16, out, lse, nsel, NULL, NULL, dws, dws_bytes, (void*)stream));
  HIP_OK(hipStreamSynchronize(stream));

  const size_t out_bytes = (size_t)B * Hq * d * sizeof(float), h_bytes = (size_t)B * Hq * 4;
  void* h_out = malloc(out_bytes);
  void* h_lse = malloc(h_bytes);
  void* h_nsel = malloc(h_bytes);
  void* h_off = malloc(off_bytes);
  void* h_idx = malloc(idx_bytes);
  if (!h_out || !h_lse || !h_nsel || !h_off || !h_idx) return 1;
  HIP_OK(hipMemcpy(h_out, out, out_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse, lse, h_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_nsel, nsel, h_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_off, offsets, off_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_idx, indices, idx_bytes, hipMemcpyDeviceToHost));
  if (!write_file(dir, "out.bin", h_out, out_bytes) || !write_file(dir, "lse.bin", h_lse, h_bytes) ||
      !write_file(dir, "nsel.bin", h_nsel, h_bytes) || !write_file(dir, "offsets.bin", h_off, off_bytes) ||
      !write_file(dir, "indices.bin", h_idx, idx_bytes)) {
    fprintf(stderr, "cannot write outputs to %s\n", dir);
    return 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  printf("abi_smoke: B=%d Hq=%d Hkv=%d N=%d K=%d L=%d T=%d stride=%d ok\n", B, Hq, Hkv, N, K, L, T, stride);
  return 0;
}
