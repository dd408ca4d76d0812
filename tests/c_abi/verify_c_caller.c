/*
 * A plain C caller of libverify_attn.so: the verify path driven through
 * include/verify_attn.h and the HIP runtime's C API alone, no Python.
 *
 *   verify_c_caller abi        host-only calls (version, status strings, workspace
 *                              size, the gate, the slot heuristic) on fake device
 *                              pointers; prints key=value lines
 *   verify_c_caller inputs FILE  writes the seeded problem's host arrays to FILE
 *                              (kv_indices, q, k_cache, v_cache), no device use
 *   verify_c_caller run FILE   one call on the GPU: uploads a seeded problem, runs
 *                              verify_attn_build_block_table, verify_attn_fwd and
 *                              verify_attn_combine on the default stream, and writes
 *                              the block table, kv_lens, out (bf16 bits) and lse to FILE
 *
 * The problem: B = 3 sequences with prefix lengths 0, 17, 100, D = 4 draft tokens,
 * 8 query heads over 2 KV heads, head dim 128, bf16 cache in pages of 4 slots drawn
 * from a shuffled 40-page pool.  Every input value comes from one splitmix64 stream
 * (seed 12345, Steele, Lea and Flood's published generator) in the order: page
 * shuffle, q, k_cache, v_cache; values are uniform in [-1, 1) rounded to bf16.  The
 * test that runs this program draws the same stream in Python and hands it to the
 * oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "verify_attn.h"

enum { B = 3, D = 4, HQ = 8, HKV = 2, DIM = 128, PAGE = 4, POOL_PAGES = 40 };
static const int32_t kPrefix[B] = {0, 17, 100};

static uint64_t splitmix64(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* uniform in [-1, 1) from the top 24 bits, rounded to bf16 (nearest even) */
static uint16_t next_bf16(uint64_t* s) {
  const float x = (float)((double)(splitmix64(s) >> 40) / 16777216.0) * 2.0f - 1.0f;
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define CHECK_HIP(call)                                                           \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)
#define CHECK_VA(call)                                                            \
  do {                                                                            \
    int s_ = (call);                                                              \
    if (s_ != VA_OK) {                                                            \
      fprintf(stderr, "%s returned %d (%s)\n", #call, s_, verify_attn_strerror(s_)); \
      exit(3);                                                                    \
    }                                                                             \
  } while (0)

static void fill_args(verify_attn_args* a, void* q, void* k, void* v, int32_t* bt,
                      int32_t max_pages, int32_t* lens, float* ws, int64_t ws_bytes,
                      void* out, float* lse) {
  memset(a, 0, sizeof(*a));
  a->struct_size = (int32_t)sizeof(verify_attn_args);
  a->batch = B;
  a->draft_len = D;
  a->hq = HQ;
  a->hkv = HKV;
  a->qk_dim = DIM;
  a->v_dim = DIM;
  a->page_size = PAGE;
  a->kv_dtype = VA_KV_BF16;
  a->sm_scale = 1.0f / sqrtf((float)DIM);
  a->k_scale = 1.0f;
  a->v_scale = 1.0f;
  a->window_left = -1;
  a->max_prefix_len = 100;
  a->num_splits = 0;
  a->q = q;
  a->q_stride_row = HQ * DIM;
  a->q_stride_head = DIM;
  a->k_cache = k;
  a->k_stride_slot = HKV * DIM;
  a->k_stride_head = DIM;
  a->v_cache = v;
  a->v_stride_slot = HKV * DIM;
  a->v_stride_head = DIM;
  a->block_table = bt;
  a->max_pages_per_seq = max_pages;
  a->prefix_lens = lens;
  a->workspace = ws;
  a->workspace_bytes = ws_bytes;
  a->out = out;
  a->o_stride_row = HQ * DIM;
  a->o_stride_head = DIM;
  a->lse = lse;
}

static int abi_checks(void) {
  char* fake = (char*)(uintptr_t)0x10000; /* 16-byte aligned, never dereferenced */
  verify_attn_args a;
  printf("abi_version=%d\n", (int)verify_attn_abi_version());
  printf("strerror_ok=%s\n", verify_attn_strerror(VA_OK));
  printf("workspace_bytes_s4=%lld\n",
         (long long)verify_attn_workspace_bytes(B, HKV, HQ, D, DIM, 4));
  printf("workspace_bytes_bad=%lld\n",
         (long long)verify_attn_workspace_bytes(B, HKV, HQ + 1, D, DIM, 4));
  fill_args(&a, fake, fake, fake, (int32_t*)fake, 26, (int32_t*)fake, (float*)fake, 1 << 20,
            fake, (float*)fake);
  printf("can_handle=%d\n", verify_attn_can_handle(&a));
  printf("num_splits_positive=%d\n", verify_attn_num_splits(&a) >= 1);
  a.draft_len = 9;
  printf("can_handle_draft9=%d\n", verify_attn_can_handle(&a));
  a.draft_len = D;
  a.qk_dim = 96;
  printf("can_handle_dim96=%d\n", verify_attn_can_handle(&a));
  a.qk_dim = DIM;
  a.q = NULL;
  printf("can_handle_null_q=%d\n", verify_attn_can_handle(&a));
  a.q = fake;
  a.workspace_bytes = 16;
  printf("fwd_small_workspace=%d\n", verify_attn_fwd(&a, NULL));
  return 0;
}

/* The seeded problem's host arrays (see the file header). */
typedef struct {
  int n_of[B], pages_of[B], total_tokens, max_pages;
  int32_t indptr[B + 1];
  int32_t* indices;
  uint16_t *q, *k, *v;
  size_t nq, nkv;
} host_problem;

static void make_inputs(host_problem* h) {
  uint64_t st = 12345;
  h->total_tokens = 0;
  h->max_pages = 0;
  for (int b = 0; b < B; ++b) {
    h->n_of[b] = kPrefix[b] + D;
    h->pages_of[b] = (h->n_of[b] + PAGE - 1) / PAGE;
    h->total_tokens += h->n_of[b];
    if (h->pages_of[b] > h->max_pages) h->max_pages = h->pages_of[b];
  }
  /* page shuffle: Fisher-Yates over the pool, draws j = next % (i + 1) for i = n-1..1 */
  int perm[POOL_PAGES];
  for (int i = 0; i < POOL_PAGES; ++i) perm[i] = i;
  for (int i = POOL_PAGES - 1; i > 0; --i) {
    const int j = (int)(splitmix64(&st) % (uint64_t)(i + 1));
    const int t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  h->indices = (int32_t*)malloc(sizeof(int32_t) * h->total_tokens);
  h->indptr[0] = 0;
  for (int b = 0, p0 = 0; b < B; ++b) {
    for (int t = 0; t < h->n_of[b]; ++t)
      h->indices[h->indptr[b] + t] = perm[p0 + t / PAGE] * PAGE + t % PAGE;
    h->indptr[b + 1] = h->indptr[b] + h->n_of[b];
    p0 += h->pages_of[b];
  }
  h->nq = (size_t)B * D * HQ * DIM;
  h->nkv = (size_t)POOL_PAGES * PAGE * HKV * DIM;
  h->q = (uint16_t*)malloc(h->nq * 2);
  h->k = (uint16_t*)malloc(h->nkv * 2);
  h->v = (uint16_t*)malloc(h->nkv * 2);
  for (size_t i = 0; i < h->nq; ++i) h->q[i] = next_bf16(&st);
  for (size_t i = 0; i < h->nkv; ++i) h->k[i] = next_bf16(&st);
  for (size_t i = 0; i < h->nkv; ++i) h->v[i] = next_bf16(&st);
}

static int dump_inputs(const char* path) {
  host_problem h;
  make_inputs(&h);
  FILE* f = fopen(path, "wb");
  if (!f) {
    perror(path);
    return 5;
  }
  fwrite(h.indices, sizeof(int32_t), (size_t)h.total_tokens, f);
  fwrite(h.q, 2, h.nq, f);
  fwrite(h.k, 2, h.nkv, f);
  fwrite(h.v, 2, h.nkv, f);
  fclose(f);
  return 0;
}

static int run(const char* path) {
  host_problem h;
  make_inputs(&h);
  const int max_pages = h.max_pages, total_tokens = h.total_tokens;
  const size_t nq = h.nq, nkv = h.nkv;
  const int32_t* indptr = h.indptr;
  const int32_t* indices = h.indices;
  const uint16_t *hq = h.q, *hk = h.k, *hv = h.v;
  void *dq, *dk, *dv, *dout;
  int32_t *dindptr, *dindices, *dbt, *dkvlens, *dprefix;
  float *dlse, *dws;
  CHECK_HIP(hipMalloc(&dq, nq * 2));
  CHECK_HIP(hipMalloc(&dk, nkv * 2));
  CHECK_HIP(hipMalloc(&dv, nkv * 2));
  CHECK_HIP(hipMalloc((void**)&dindptr, sizeof(int32_t) * (B + 1)));
  CHECK_HIP(hipMalloc((void**)&dindices, sizeof(int32_t) * total_tokens));
  CHECK_HIP(hipMalloc((void**)&dbt, sizeof(int32_t) * B * max_pages));
  CHECK_HIP(hipMalloc((void**)&dkvlens, sizeof(int32_t) * B));
  CHECK_HIP(hipMalloc((void**)&dprefix, sizeof(kPrefix)));
  CHECK_HIP(hipMalloc(&dout, nq * 2));
  CHECK_HIP(hipMalloc((void**)&dlse, sizeof(float) * B * D * HQ));
  CHECK_HIP(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, nkv * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, nkv * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dindptr, indptr, sizeof(int32_t) * (B + 1), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dindices, indices, sizeof(int32_t) * total_tokens, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dprefix, kPrefix, sizeof(kPrefix), hipMemcpyHostToDevice));

  CHECK_VA(verify_attn_build_block_table(dindptr, dindices, B, PAGE, max_pages, dbt, dkvlens, NULL));
  verify_attn_args a;
  fill_args(&a, dq, dk, dv, dbt, max_pages, dprefix, NULL, 0, dout, dlse);
  const int32_t splits = verify_attn_num_splits(&a);
  if (splits < 1) {
    fprintf(stderr, "verify_attn_num_splits returned %d\n", (int)splits);
    return 4;
  }
  const int64_t ws_bytes = verify_attn_workspace_bytes(B, HKV, HQ, D, DIM, splits);
  CHECK_HIP(hipMalloc((void**)&dws, (size_t)ws_bytes));
  a.workspace = dws;
  a.workspace_bytes = ws_bytes;
  a.num_splits = splits;
  CHECK_VA(verify_attn_fwd(&a, NULL));
  CHECK_VA(verify_attn_combine(&a, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  int32_t* hbt = (int32_t*)malloc(sizeof(int32_t) * B * max_pages);
  int32_t hlens[B];
  uint16_t* hout = (uint16_t*)malloc(nq * 2);
  float* hlse = (float*)malloc(sizeof(float) * B * D * HQ);
  CHECK_HIP(hipMemcpy(hbt, dbt, sizeof(int32_t) * B * max_pages, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hlens, dkvlens, sizeof(hlens), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hout, dout, nq * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hlse, dlse, sizeof(float) * B * D * HQ, hipMemcpyDeviceToHost));
  FILE* f = fopen(path, "wb");
  if (!f) {
    perror(path);
    return 5;
  }
  const int32_t header[3] = {B, max_pages, splits};
  fwrite(header, sizeof(header), 1, f);
  fwrite(hbt, sizeof(int32_t), (size_t)B * max_pages, f);
  fwrite(hlens, sizeof(hlens), 1, f);
  fwrite(hout, 2, nq, f);
  fwrite(hlse, sizeof(float), (size_t)B * D * HQ, f);
  fclose(f);
  printf("splits=%d\n", (int)splits);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "abi") == 0) return abi_checks();
  if (argc >= 3 && strcmp(argv[1], "inputs") == 0) return dump_inputs(argv[2]);
  if (argc >= 3 && strcmp(argv[1], "run") == 0) return run(argv[2]);
  fprintf(stderr, "usage: %s abi | inputs FILE | run FILE\n", argv[0]);
  return 1;
}
