// Block-table scatter: token-level ragged slot lists -> [B, max_pages] page ids.
//
// At topk = 1 the slots of a page are consecutive (PR #5168, "Support Page Size > 1
// (when top k = 1) for FA3 Spec Decode", reviewer comment), so the page of token t
// is the slot of the page's first token divided by P.  One thread per table entry
// reads only page-leading entries and needs no per-token scratch (PR #23146 builds
// the same table without a bs x max_context_len buffer).  Integer only.

#include "va_internal.h"

namespace va {

struct BlockTableParams {
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int32_t batch, lg_page, max_pages;
  int32_t* block_table;
  int32_t* kv_lens;
};

__global__ __launch_bounds__(256) void block_table_kernel(BlockTableParams P) {
  const int32_t* __restrict__ kv_indptr = P.kv_indptr;
  const int32_t* __restrict__ kv_indices = P.kv_indices;
  const int32_t batch = P.batch, lg_page = P.lg_page, max_pages = P.max_pages;
  int32_t* __restrict__ block_table = P.block_table;
  int32_t* __restrict__ kv_lens = P.kv_lens;
  const int b = blockIdx.y;
  const int pg = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch || pg >= max_pages) return;
  const int start = kv_indptr[b];
  const int n = kv_indptr[b + 1] - start;
  const int npages = (n + (1 << lg_page) - 1) >> lg_page;
  int v = 0;
  if (pg < npages) v = kv_indices[start + (pg << lg_page)] >> lg_page;
  block_table[(int64_t)b * max_pages + pg] = v;
  if (pg == 0 && kv_lens) kv_lens[b] = n;
}

int launch_block_table(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                       int lg_page, int32_t max_pages, int32_t* block_table, int32_t* kv_lens,
                       hipStream_t stream) {
  if (batch > 65535) return VA_EUNSUPPORTED;
  dim3 grid((max_pages + 255) / 256, batch);
  const BlockTableParams p{kv_indptr, kv_indices, batch, lg_page, max_pages, block_table, kv_lens};
  return launch_kernel(reinterpret_cast<const void*>(&block_table_kernel), grid, dim3(256), p,
                       stream);
}

// Sliding-window pool slots (PR #23146 page-table code: full-pool locations are
// translated to the window pool before the table transform): out[i] =
// full_to_swa[in[i]], one thread per entry.
struct TranslateParams {
  const int32_t* in;
  int64_t n;
  const int32_t* map;
  int32_t* out;
};

__global__ __launch_bounds__(256) void translate_slots_kernel(TranslateParams P) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < P.n) P.out[i] = P.map[P.in[i]];
}

int launch_translate_slots(const int32_t* in, int64_t n, const int32_t* full_to_swa, int32_t* out,
                           hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return VA_EUNSUPPORTED;
  const TranslateParams p{in, n, full_to_swa, out};
  return launch_kernel(reinterpret_cast<const void*>(&translate_slots_kernel),
                       dim3((unsigned)blocks), dim3(256), p, stream);
}

}  // namespace va
