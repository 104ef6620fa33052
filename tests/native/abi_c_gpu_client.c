/* A plain C11 program that runs the whole path through include/segpaged.h with device memory
 * it allocates itself (hipMalloc; no Python, no torch): build, plan, attention, check.
 *   abi_c_gpu_client IN OUT
 * IN (little-endian): int32 dtype, B, Hq, Hkv, D, P; int32 ctx_len[B], q_len[B];
 * int32 policy[Hkv][3]; float32 scale; then K and V [sum(ctx_len)][Hkv][D] and
 * Q [sum(q_len)][Hq][D] as raw elements (2-byte bf16 or 4-byte float32).
 * OUT: O [sum(q_len)][Hq][D], raw elements of the same type. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "segpaged.h"

#define CHECK_HIP(x)                                              \
  do {                                                            \
    if ((x) != hipSuccess) {                                      \
      fprintf(stderr, "HIP error at line %d\n", __LINE__);        \
      return 2;                                                   \
    }                                                             \
  } while (0)
#define CHECK_SP(x)                                                                   \
  do {                                                                                \
    sp_status s_ = (x);                                                               \
    if (s_ != SP_OK) {                                                                \
      fprintf(stderr, "%s at line %d\n", segpaged_status_string(s_), __LINE__);      \
      return 3;                                                                       \
    }                                                                                 \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) return 1;
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) return 1;
  int32_t hdr[6];
  if (!read_all(in, hdr, sizeof(hdr))) return 1;
  const sp_dtype dtype = (sp_dtype)hdr[0];
  const int32_t B = hdr[1], Hq = hdr[2], Hkv = hdr[3], D = hdr[4], P = hdr[5];
  if (B < 1 || Hkv < 1 || Hq < Hkv || D < 1 || P < 1) return 1;
  const size_t es = dtype == SP_BF16 ? 2 : 4;
  int32_t* ctx = malloc(sizeof(int32_t) * (size_t)B);
  int32_t* q = malloc(sizeof(int32_t) * (size_t)B);
  sp_head_policy* pol = malloc(sizeof(sp_head_policy) * (size_t)Hkv);
  float scale = 0.f;
  if (!read_all(in, ctx, sizeof(int32_t) * (size_t)B) ||
      !read_all(in, q, sizeof(int32_t) * (size_t)B) ||
      !read_all(in, pol, sizeof(sp_head_policy) * (size_t)Hkv) ||
      !read_all(in, &scale, sizeof(float)))
    return 1;
  size_t T = 0, Tq = 0;
  for (int32_t b = 0; b < B; ++b) {
    T += (size_t)ctx[b];
    Tq += (size_t)q[b];
  }
  const size_t kv_bytes = T * (size_t)Hkv * (size_t)D * es;
  const size_t q_bytes = Tq * (size_t)Hq * (size_t)D * es;
  void* hk = malloc(kv_bytes + 1);
  void* hv = malloc(kv_bytes + 1);
  void* hq = malloc(q_bytes + 1);
  void* ho = malloc(q_bytes + 1);
  if (!read_all(in, hk, kv_bytes) || !read_all(in, hv, kv_bytes) || !read_all(in, hq, q_bytes))
    return 1;
  fclose(in);

  int64_t n_virt = 0;
  CHECK_SP(segpaged_plan_pages(B, ctx, q, Hkv, pol, P, &n_virt));
  const int64_t n_phys = n_virt > 0 ? n_virt : 1;
  int32_t* free_pages = malloc(sizeof(int32_t) * (size_t)n_phys);
  for (int64_t i = 0; i < n_phys; ++i) free_pages[i] = (int32_t)(n_phys - 1 - i);

  void *dk, *dv, *dq, *dout, *kp, *vp, *ws;
  int32_t* tables;
  const size_t n_tab = (size_t)B * (size_t)Hkv * 8, n_kl = (size_t)B * (size_t)Hkv;
  const size_t pool_bytes = (size_t)n_phys * (size_t)P * (size_t)D * es;
  CHECK_HIP(hipMalloc(&dk, kv_bytes + 16));
  CHECK_HIP(hipMalloc(&dv, kv_bytes + 16));
  CHECK_HIP(hipMalloc(&dq, q_bytes + 16));
  CHECK_HIP(hipMalloc(&dout, q_bytes + 16));
  CHECK_HIP(hipMalloc(&kp, pool_bytes));
  CHECK_HIP(hipMalloc(&vp, pool_bytes));
  CHECK_HIP(hipMalloc((void**)&tables, sizeof(int32_t) * (n_tab + n_kl + (size_t)n_phys)));
  CHECK_HIP(hipMemcpy(dk, hk, kv_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, kv_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dq, hq, q_bytes, hipMemcpyHostToDevice));
  int32_t* seg = tables;
  int32_t* kvl = tables + n_tab;
  int32_t* v2p = tables + n_tab + n_kl;
  CHECK_SP(segpaged_build(dtype, B, Hkv, D, P, ctx, q, pol, dk, dv, free_pages, n_phys, n_phys,
                          kp, vp, seg, kvl, v2p, NULL));
  size_t ws_bytes = 0;
  CHECK_SP(segpaged_attention_workspace_size(dtype, B, Hq, Hkv, D, P, ctx, q, pol, &ws_bytes));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_SP(segpaged_attention_plan(dtype, B, Hq, Hkv, D, P, ctx, q, pol, ws, ws_bytes, NULL));
  CHECK_SP(segpaged_attention(dtype, B, Hq, Hkv, D, P, ctx, q, pol, dq, kp, vp, n_phys, seg, kvl,
                              v2p, scale, dout, ws, ws_bytes, NULL));
  CHECK_SP(segpaged_attention_check(ws, ws_bytes, NULL));
  CHECK_HIP(hipMemcpy(ho, dout, q_bytes, hipMemcpyDeviceToHost));
  FILE* out = fopen(argv[2], "wb");
  if (out == NULL || fwrite(ho, 1, q_bytes, out) != q_bytes) return 1;
  fclose(out);
  hipFree(dk);
  hipFree(dv);
  hipFree(dq);
  hipFree(dout);
  hipFree(kp);
  hipFree(vp);
  hipFree(tables);
  hipFree(ws);
  printf("ok %lld pages, %zu bytes of workspace\n", (long long)n_virt, ws_bytes);
  return 0;
}
