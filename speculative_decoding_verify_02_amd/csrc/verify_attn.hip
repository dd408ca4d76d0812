// C-ABI entry points: argument checks, the static-shape gate, split planning and
// workspace sizing.  Every decision here reads host scalars only, so a call can be
// captured into a HIP graph (the split-KV page's can_handle() gate and its
// max-batch-keyed scratch follow the same rule).

#include <math.h>
#include <string.h>

#include <mutex>

#include "va_internal.h"

namespace va {

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte offsets of a slot row and of the last KV head inside it fit in 32 bits (the
// tile kernel adds slot * slot stride as one 32 x 32 -> 64-bit product and keeps the
// in-row offset in 32 bits).
bool slot_offsets_fit_32(const verify_attn_args* a) {
  const int64_t lim = (int64_t)1 << 31;
  return a->k_stride_slot * 2 < lim && a->v_stride_slot * 2 < lim &&
         ((int64_t)a->hkv * a->k_stride_head + a->qk_dim) * 2 < lim &&
         ((int64_t)a->hkv * a->v_stride_head + a->v_dim) * 2 < lim;
}

bool supported_dims(int qk, int v) {
  return (qk == 128 && v == 128) || (qk == 256 && v == 256) || (qk == 576 && v == 512);
}

// Attended prefix length bound: the union of the draft rows' windows starts at
// max(0, L - W), so at most min(L, W) prefix keys are visible.
int max_attended_prefix(int max_prefix_len, int window_left) {
  return window_left >= 0 ? (max_prefix_len < window_left ? max_prefix_len : window_left)
                          : max_prefix_len;
}

constexpr int kMaxSlots = 256;  // heuristic cap on partial slots per (sequence, KV head)

// Split heuristic: how many key ranges (grid rows) and partial slots.  The grid
// is one full round of workgroups across the chip (per_cu x CUs, with head_groups
// workgroups per range), and the device cuts the keys of all sequences into that
// many equal ranges.  The slot count bounds the pieces of one sequence: about
// twice its even share of the ranges, so the bound rarely limits the balance,
// and never more than a sequence of the host's maximum length can need.
void heuristic_grid(int batch, int head_groups, int maxlen, int min_q, int cus, int per_cu,
                    int* nwy, int* slots) {
  const long long rows = ((long long)cus * per_cu + head_groups - 1) / head_groups;
  *nwy = (int)(rows < 1 ? 1 : (rows > 65535 ? 65535 : rows));
  if (batch <= 0 || maxlen <= 0) {
    *slots = 1;
    return;
  }
  long long s = (2LL * *nwy + batch - 1) / batch + 1;
  const long long s_need = (long long)(maxlen - 1) / min_q + 2;  // pieces of a maxlen sequence
  if (s > s_need) s = s_need;
  if (s > kMaxSlots) s = kMaxSlots;
  *slots = (int)(s < 2 ? 2 : s);
}

}  // namespace

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int make_plan(const verify_attn_args* a, Plan* p, bool check_pointers) {
  if (!a || a->struct_size != (int32_t)sizeof(verify_attn_args)) return VA_EINVAL;
  // extensions: a tree needs its mask, takes uniform rows and no window
  if ((a->draft_slots == nullptr) != (a->tree_mask == nullptr)) return VA_EINVAL;
  if (!(a->logit_cap >= 0.f) || !isfinite(a->logit_cap)) return VA_EINVAL;
  if (a->draft_slots && (a->qo_indptr || a->window_left >= 0)) return VA_EUNSUPPORTED;
  if (a->batch < 0 || a->draft_len < 1 || a->hq < 1 || a->hkv < 1 || a->max_prefix_len < 0 ||
      a->num_splits < 0 || a->window_left < -1 || a->max_pages_per_seq < 1)
    return VA_EINVAL;
  if (a->hq % a->hkv != 0) return VA_EINVAL;
  if (!(isfinite(a->sm_scale) && isfinite(a->k_scale) && isfinite(a->v_scale)))
    return VA_EINVAL;
  if (a->kv_dtype != VA_KV_BF16 && a->kv_dtype != VA_KV_FP8_E4M3FN) return VA_EINVAL;
  if (a->kv_dtype == VA_KV_BF16 && (a->k_scale != 1.0f || a->v_scale != 1.0f))
    return VA_EINVAL;
  if (a->draft_len > 8) return VA_EUNSUPPORTED;
  if (!supported_dims(a->qk_dim, a->v_dim)) return VA_EUNSUPPORTED;
  if (!is_pow2(a->page_size) || a->page_size > 1024) return VA_EUNSUPPORTED;
  const int group = a->hq / a->hkv;
  const int rows = group * a->draft_len;
  if (rows > kMaxRows) return VA_EUNSUPPORTED;
  // the combine's grid has hkv and batch as its y and z dimensions (at most 65535
  // each): the launchers refuse more, so the gate does too
  if (a->batch > 65535 || a->hkv > 65535) return VA_EUNSUPPORTED;

  if (a->batch > 0) {
    if (check_pointers && (!a->q || !a->k_cache || !a->v_cache || !a->block_table ||
                           !a->prefix_lens || !a->workspace || !a->out))
      return VA_EINVAL;
    const int eb = a->kv_dtype == VA_KV_FP8_E4M3FN ? 1 : 2;
    // 16-byte vector loads of q / K / V rows need 16-byte aligned rows
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) ||
        !aligned16(a->workspace))
      return VA_EINVAL;
    if (a->q_stride_row <= 0 || a->q_stride_head <= 0 || (a->q_stride_row % 8) ||
        (a->q_stride_head % 8))
      return VA_EINVAL;
    const int64_t kq = 16 / eb;
    if (a->k_stride_slot <= 0 || a->k_stride_head <= 0 || (a->k_stride_slot % kq) ||
        (a->k_stride_head % kq) || a->v_stride_slot <= 0 || a->v_stride_head <= 0 ||
        (a->v_stride_slot % kq) || (a->v_stride_head % kq))
      return VA_EINVAL;
    if (a->o_stride_row <= 0 || a->o_stride_head <= 0) return VA_EINVAL;
    if (a->k_stride_head < a->qk_dim || a->v_stride_head < a->v_dim) return VA_EINVAL;
    // kernels form a slot row's address as slot * (slot stride in bytes), 32 x 32 bits
    if (a->k_stride_slot * eb >= ((int64_t)1 << 32) || a->v_stride_slot * eb >= ((int64_t)1 << 32))
      return VA_EUNSUPPORTED;
  }

  p->group = group;
  p->rows = rows;
  const bool fp8 = a->kv_dtype == VA_KV_FP8_E4M3FN;
  int head_groups = a->hkv, per_cu = 1;
  // the MLA kernel reads V as the first v_dim bytes of the K row it already holds, so
  // it serves only a V cache that is that view of the K cache; a separate V cache of
  // the same shape takes the generic kernel
  const bool v_is_k_view = a->v_cache == a->k_cache && a->v_stride_slot == a->k_stride_slot &&
                           a->v_stride_head == a->k_stride_head;
  if (fp8 && a->qk_dim == 576 && rows <= 64 && v_is_k_view) {
    p->kind = kMlaFp8;                      // one workgroup per (head, split), 4 row-group waves
    p->rt = 1;
    p->nrg = 4;
    p->ntl = 1;
    p->hpc = 1;
  } else if (!fp8 && a->qk_dim == 256 && a->v_dim == 256 && rows <= 64 &&
             slot_offsets_fit_32(a)) {
    // wide bf16 heads: whole-slot-row tiles (d = 128 streams better per wave)
    p->kind = kTile;
    p->rt = 1;
    p->nrg = (rows + 15) / 16;
    if (p->nrg == 3) p->nrg = 4;
    p->ntl = 1;
    const int max_hpc = 4 / p->nrg;  // at most 4 waves of d = 256 rows
    p->hpc = 1;
    while (p->hpc * 2 <= max_hpc && a->hkv % (p->hpc * 2) == 0) p->hpc *= 2;
    head_groups = a->hkv / p->hpc;
    // one workgroup per CU: three blocks in flight in registers take a wave's whole
    // register file
    per_cu = 1;
  } else {
    p->kind = kGeneric;
    p->rt = (rows <= 16) ? 1 : (a->v_dim <= 256 ? 2 : 1);
    const int tiles = (rows + 15) / 16;
    const int groups = (tiles + p->rt - 1) / p->rt;
    p->nrg = groups <= 1 ? 1 : (groups <= 2 ? 2 : (groups <= 4 ? 4 : 0));
    if (p->nrg == 0) return VA_EUNSUPPORTED;
    // the remaining waves of a workgroup cover more KV heads of the same tokens, then
    // interleave tokens of one head.  bf16 d = 128 takes at most 2 heads (so 2 token
    // lanes each): against 4 heads, with the non-temporal KV loads, the long-context
    // batch went 358.8 -> 344.6 us, with a 4096-key window 97.0 -> 87.1 us, 4 KV heads
    // 196 -> 186.6 us and the Llama-8B shape 17.7 -> 14.8 us; fp8 d = 128 keeps 4
    // (206 us against 212 at 2)
    const int free_waves = kWaves / p->nrg;
    const int cap = (!fp8 && a->qk_dim == 128 && free_waves > 2) ? 2 : free_waves;
    p->hpc = a->hkv >= cap ? cap : (a->hkv >= 2 && cap >= 2 ? 2 : 1);
    p->ntl = free_waves / p->hpc;
    head_groups = (a->hkv + p->hpc - 1) / p->hpc;
    // fp8 d = 128 with one row tile: two workgroups per CU; bf16 d = 128 one (with two
    // heads per workgroup that beat two per CU: long-context batch 344.0 -> 336.3 us,
    // Llama-8B shape call 23.4 -> 20.4 us, window 87.5 -> 85.2 us; fp8 at one per CU
    // 208 -> 285 us)
    per_cu = (a->qk_dim == 128 && p->rt == 1 && fp8) ? 2 : 1;
  }
  p->hg = head_groups;
  p->lg_page = ilog2(a->page_size);
  p->max_leff = max_attended_prefix(a->max_prefix_len, a->window_left);
  // fewest keys per workgroup: a few blocks of the kernel's main loop
  p->min_q = p->kind == kMlaFp8 ? 128 : (p->kind == kTile ? 64 : 64);
  // fixed cost of a piece in keys of the main loop (q load, the first block's memory
  // latency, the partial write), from per-wave timings of one- and two-piece ranges
  p->piece_cost = p->kind == kMlaFp8 ? 704 : (p->kind == kTile ? 80 : 32);
  const long long maxlen = (long long)p->max_leff + a->draft_len;
  const int maxlen_i = maxlen > INT32_MAX ? INT32_MAX : (int)maxlen;
  int nwy = 1, slots = 1;
  heuristic_grid(a->batch, head_groups, maxlen_i, p->min_q, device_cu_count(), per_cu, &nwy, &slots);
  p->slots = a->num_splits > 0 ? a->num_splits : slots;
  // one slot: grid row y takes all of sequence y
  p->nwy = p->slots == 1 ? (a->batch > 0 ? a->batch : 1) : nwy;
  if (p->nwy > 65535) return VA_EUNSUPPORTED;
  p->ws_o_floats = (int64_t)a->batch * a->hkv * p->slots * rows * a->v_dim;
  p->ws_cnt_floats = p->ws_o_floats + (int64_t)a->batch * a->hkv * p->slots * rows;
  return VA_OK;
}

// Workspace of the allocation-free entry point: one array per device, loaded with the
// library's code object and held until the process ends.  Its host-side name is only a
// handle: kernels receive the device address hipGetSymbolAddress gives for the current
// device (each device holds its own copy at its own address).
constexpr int64_t kStaticScratchBytes = VERIFY_ATTN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per device; NULL if
// the runtime cannot give it.
void* static_scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

}  // namespace

}  // namespace va

extern "C" {

int32_t verify_attn_abi_version(void) { return 2; }

const char* verify_attn_strerror(int status) {
  switch (status) {
    case VA_OK: return "ok";
    case VA_EINVAL: return "invalid argument";
    case VA_EUNSUPPORTED: return "unsupported shape or dtype (caller should fall back)";
    case VA_EWORKSPACE: return "workspace too small";
    case VA_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int64_t verify_attn_workspace_bytes(int32_t batch, int32_t hkv, int32_t hq, int32_t draft_len,
                                    int32_t v_dim, int32_t num_splits) {
  if (batch < 0 || hkv < 1 || hq < 1 || hq % hkv || draft_len < 1 || v_dim < 1 || num_splits < 1)
    return -1;
  const int64_t rows = (int64_t)(hq / hkv) * draft_len;
  return ((int64_t)batch * hkv * num_splits * rows * ((int64_t)v_dim + 1) + batch) * 4;
}

// Copies the caller's arguments into a full current-version struct: a version 1
// caller's struct ends before the extension fields, which then read as off.
static int load_args(const verify_attn_args* in, verify_attn_args* out) {
  if (!in) return VA_EINVAL;
  const int32_t sz = in->struct_size;
  if (sz != (int32_t)sizeof(verify_attn_args) && sz != VERIFY_ATTN_ARGS_V1_SIZE) return VA_EINVAL;
  memset(out, 0, sizeof(*out));
  memcpy(out, in, (size_t)sz);
  out->struct_size = (int32_t)sizeof(verify_attn_args);
  return VA_OK;
}

int32_t verify_attn_num_splits(const verify_attn_args* args) {
  va::Plan p;
  verify_attn_args a;
  if (load_args(args, &a) != VA_OK) return -1;
  a.num_splits = 0;  // the heuristic's choice, whatever the caller asked for
  return va::make_plan(&a, &p, /*check_pointers=*/false) == VA_OK ? p.slots : -1;
}

int verify_attn_can_handle(const verify_attn_args* args) {
  va::Plan p;
  verify_attn_args a;
  const int st = load_args(args, &a);
  return st != VA_OK ? st : va::make_plan(&a, &p, true);
}

static int check_workspace(const verify_attn_args* a, const va::Plan& p) {
  const int64_t need = verify_attn_workspace_bytes(a->batch, a->hkv, a->hq, a->draft_len,
                                                   a->v_dim, p.slots);
  return (need < 0 || a->workspace_bytes < need) ? VA_EWORKSPACE : VA_OK;
}

int verify_attn_fwd(const verify_attn_args* args, void* stream) {
  va::Plan p;
  verify_attn_args a;
  int st = load_args(args, &a);
  if (st != VA_OK || (st = va::make_plan(&a, &p, true)) != VA_OK) return st;
  if ((st = check_workspace(&a, p)) != VA_OK) return st;
  // launched even when the host bound says no prefix is attended: the device lengths
  // decide what each workgroup covers
  if (a.batch == 0) return VA_OK;
  return va::launch_splitkv_fwd(&a, p, reinterpret_cast<hipStream_t>(stream));
}

int verify_attn_combine(const verify_attn_args* args, void* stream) {
  va::Plan p;
  verify_attn_args a;
  int st = load_args(args, &a);
  if (st != VA_OK || (st = va::make_plan(&a, &p, true)) != VA_OK) return st;
  if ((st = check_workspace(&a, p)) != VA_OK) return st;
  if (a.batch == 0) return VA_OK;
  return va::launch_combine(&a, p, reinterpret_cast<hipStream_t>(stream));
}

int verify_attn_fwd_combine_noalloc(const verify_attn_args* args, void* stream) {
  verify_attn_args a;
  int st = load_args(args, &a);
  if (st != VA_OK) return st;
  // the caller's workspace fields are ignored.  The argument checks run before any HIP
  // call, with a non-null 256-byte aligned stand-in for the array's address (the only
  // workspace properties make_plan checks); the real address replaces it before launch.
  a.workspace = reinterpret_cast<float*>((uintptr_t)256);
  a.workspace_bytes = va::kStaticScratchBytes;
  va::Plan p;
  if ((st = va::make_plan(&a, &p, true)) != VA_OK) return st;
  if (a.batch == 0) return VA_OK;
  // the largest slot count the array holds, at most the one asked for (or the heuristic's)
  const int64_t per_slot = verify_attn_workspace_bytes(a.batch, a.hkv, a.hq, a.draft_len,
                                                       a.v_dim, 1) - (int64_t)a.batch * 4;
  const int64_t fit = per_slot > 0 ? (va::kStaticScratchBytes - (int64_t)a.batch * 4) / per_slot : 0;
  if (fit < 1) return VA_EWORKSPACE;
  if (a.num_splits > 0 && a.num_splits > fit) return VA_EWORKSPACE;
  if (a.num_splits == 0 && p.slots > fit) {
    a.num_splits = (int32_t)fit;
    if ((st = va::make_plan(&a, &p, true)) != VA_OK) return st;
  }
  if ((st = check_workspace(&a, p)) != VA_OK) return st;
  void* ptr = va::static_scratch_ptr();
  if (!ptr) return VA_EHIP;
  a.workspace = static_cast<float*>(ptr);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = va::launch_splitkv_fwd(&a, p, s)) != VA_OK) return st;
  return va::launch_combine(&a, p, s);
}

int verify_attn_translate_slots(const int32_t* in, int64_t n, const int32_t* full_to_swa,
                                int64_t map_len, int32_t* out, void* stream) {
  if (n < 0 || map_len < 1) return VA_EINVAL;
  if (n == 0) return VA_OK;
  if (!in || !full_to_swa || !out) return VA_EINVAL;
  return va::launch_translate_slots(in, n, full_to_swa, out, reinterpret_cast<hipStream_t>(stream));
}

int verify_attn_build_block_table(const int32_t* kv_indptr, const int32_t* kv_indices,
                                  int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                  int32_t* block_table, int32_t* kv_lens, void* stream) {
  if (batch < 0 || max_pages_per_seq < 1) return VA_EINVAL;
  if (!va::is_pow2(page_size) || page_size > 1024) return VA_EUNSUPPORTED;
  if (batch == 0) return VA_OK;
  if (!kv_indptr || !kv_indices || !block_table) return VA_EINVAL;
  return va::launch_block_table(kv_indptr, kv_indices, batch, va::ilog2(page_size),
                                max_pages_per_seq, block_table, kv_lens,
                                reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
