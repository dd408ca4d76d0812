// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "verify_attn.h"

namespace va {

// 16-byte MFMA operand of 8 bf16 and the 4-float accumulator of a 16x16 tile.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;  // 16x16x16 MFMA operand

constexpr int kTokBlock = 32;   // prefix tokens one wave handles per main-loop step
constexpr int kWaves = 4;       // waves per split-KV workgroup
constexpr int kMaxRows = 128;   // G*D rows one workgroup can hold

// Everything the kernels need, resolved on the host from verify_attn_args.
enum KernelKind { kGeneric = 0, kTile = 1, kMlaFp8 = 2 };

struct Plan {
  int kind;         // which split-KV kernel serves the call (KernelKind)
  int rows;         // G * D query rows per KV head
  int group;        // G
  int rt;           // 16-row MFMA tiles per wave (1 or 2)
  int nrg;          // row groups of one KV head (1, 2, 4)
  int ntl;          // token lanes: waves that interleave one (head, row group)'s blocks
  int hpc;          // KV heads per workgroup; hpc * nrg * ntl = 4 waves
  int lg_page;      // log2(page_size)
  int splits;       // split slots per (sequence, KV head)
  int chunk;        // prefix tokens per split (multiple of kTokBlock)
  int max_leff;     // max over sequences of the attended prefix length
  int64_t ws_o_floats;  // offset of partial LSEs in the workspace (floats)
};

// Split-KV kernel parameters (strides in bytes), resolved from verify_attn_args.
struct FwdParams {
  const uint8_t* q;  // bf16
  int64_t q_srow, q_shead;   // bytes
  const uint8_t* k;
  int64_t k_sslot, k_shead;  // bytes
  const uint8_t* v;
  int64_t v_sslot, v_shead;  // bytes
  const int32_t* bt;
  int32_t max_pages;
  const int32_t* prefix_lens;
  float* part_o;
  float* part_lse;
  int hkv, group, draft, rows, lg_page, window, splits, chunk;
  float c_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
};

// Validates args (host only) and fills the plan.  Returns a VA_ status.  Pointer
// checks (null, alignment) are skipped when check_pointers is false.
int make_plan(const verify_attn_args* a, Plan* plan, bool check_pointers);

// Kernel launchers (one per translation unit).
int launch_block_table(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                       int lg_page, int32_t max_pages, int32_t* block_table, int32_t* kv_lens,
                       hipStream_t stream);
int launch_splitkv_fwd(const verify_attn_args* a, const Plan& p, hipStream_t stream);
// bf16 heads with qk_dim = v_dim in {128, 256}: whole-slot-row tiles shared by
// hpc heads x nrg row groups.
int launch_splitkv_tile(const FwdParams& fp, int d, int hpc, int nrg, dim3 grid, hipStream_t stream);
// fp8 MLA heads (qk_dim 576, v_dim 512 = first 512 of the K row), <= 64 rows per head.
int launch_splitkv_mla_fp8(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t stream);
int launch_combine(const verify_attn_args* a, const Plan& p, hipStream_t stream);

// Compute-unit count of the current device (cached per device).
int device_cu_count();

// Launches a kernel taking one by-value parameter struct.  The status comes from this
// launch alone (not from the runtime's sticky last-error slot, which other code in
// the process may have left set).
template <typename Params>
inline int launch_kernel(const void* fn, dim3 grid, dim3 block, const Params& params,
                         hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&params)};
  return hipLaunchKernel(fn, grid, block, args, 0, stream) == hipSuccess ? VA_OK : VA_EHIP;
}

}  // namespace va
