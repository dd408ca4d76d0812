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
  int hg;           // head groups: workgroups along grid x
  int lg_page;      // log2(page_size)
  int slots;        // partial slots per (sequence, KV head): the split count S
  int nwy;          // workgroups along grid y (token ranges)
  int min_q;        // fewest tokens one workgroup is given
  int piece_cost;   // fixed cost of one piece, in keys of the kernel's main loop
  int max_leff;     // host bound of the attended prefix length
  int64_t ws_o_floats;    // offset of partial LSEs in the workspace (floats)
  int64_t ws_cnt_floats;  // offset of the per-sequence piece counts (int32)
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
  int32_t* counts;   // [B] pieces written per sequence
  int batch, hkv, group, draft, rows, lg_page, window;
  int slots, min_q;
  int piece_cost;  // fixed cost of one piece in keys (cost-balanced partition)
  float c_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
  // extensions (NULL / 0: off)
  const int32_t* qo_indptr;    // [B+1] ragged rows: sequence b has rows qo[b] .. qo[b+1]-1
  const int32_t* draft_slots;  // [B, D] tree verify: slot of draft key j
  const uint8_t* tree_mask;    // [B, D, D] tree verify: row i sees draft key j
  float logit_cap;             // > 0: natural-log scores s -> cap * tanh(s / cap)
};

// Read-only int32 tables (prefix lengths, row offsets, block table) through the constant address
// space: a wave-uniform index then becomes a scalar load.
__device__ __forceinline__ int load_ro(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Draft rows of sequence b and the q/out row of its first one (scalar loads for a
// uniform b: their waits never count the vector loads in flight).
__device__ __forceinline__ int seq_rows(const FwdParams& P, int b) {
  return P.qo_indptr ? load_ro(P.qo_indptr, b + 1) - load_ro(P.qo_indptr, b) : P.draft;
}
__device__ __forceinline__ int seq_row0(const FwdParams& P, int b) {
  return P.qo_indptr ? load_ro(P.qo_indptr, b) : b * P.draft;
}

// Slot of key t of sequence b: prefix keys (and, at topk = 1, draft keys) through
// the block table; in tree verify the D draft keys t >= L through draft_slots.
__device__ __forceinline__ int key_slot(const FwdParams& P, const int32_t* bt_row, int b, int L,
                                        int t, int lg, int pmask) {
  if (P.draft_slots && t >= L) return P.draft_slots[b * P.draft + (t - L)];
  return (bt_row[t >> lg] << lg) | (t & pmask);
}

// Tree verify: the draft keys row i of sequence b sees, one bit per draft key.
__device__ __forceinline__ uint32_t tree_bits(const FwdParams& P, int b, int i) {
  uint32_t m = 0;
  const uint8_t* r = P.tree_mask + ((int64_t)b * P.draft + i) * P.draft;
  for (int jj = 0; jj < P.draft; ++jj) m |= (r[jj] ? 1u : 0u) << jj;
  return m;
}

// Key t visible to a row with key range [lo, hi] (tree verify: draft keys t >= L by
// the row's bits).
__device__ __forceinline__ bool key_ok(int t, int lo, int hi, int L, uint32_t bits, bool tree) {
  return (t >= lo) && (t <= hi) && (!tree || t < L || ((bits >> (t - L)) & 1u));
}

// Logit cap on a score in the exp2 domain: x = s * log2(e) with s natural-log, so the
// capped value is cap * log2(e) * tanh(s / cap).  tanh(y) = (e - 1) / (e + 1) with
// e = exp(2y) = 2^(2x / cap); |2x / cap| is clamped at 60, where tanh is 1 in fp32.
// The absolute error of the capped score is a few ulp of cap.
__device__ __forceinline__ float cap_log2(float x, float cap) {
  constexpr float kLog2e = 1.44269504088896340736f;
  const float z = fminf(fmaxf(x * (2.f / cap), -60.f), 60.f);
  const float e = __builtin_amdgcn_exp2f(z);
  return (cap * kLog2e) * (e - 1.f) * __builtin_amdgcn_rcpf(e + 1.f);
}

// Max and sum over the four lanes n, n + 16, n + 32, n + 48 of a wave (one score row
// spread over the four 16-lane rows of an MFMA output), with gfx950's row swaps:
// permlane16_swap of x with itself leaves x of rows {0, 1} (and {2, 3}) in the two
// results of each lane of the pair, permlane32_swap those of rows {0, 2} and {1, 3}.
// Every lane of the group gets the bit-identical result.  No LDS round trip.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ---------------------------------------------------------------------------
// Work partition of the split-KV pass (device side, identical in every wave).
//
// Sequence b owns len_b = (L_b - lo_b) + n_b keys: its attended prefix [lo_b, L_b)
// (lo_b = max(0, L_b - W) with a left window W, else 0) and then its n_b draft keys
// (n_b = D, or qo[b+1] - qo[b] with ragged rows), which sit in the paged cache
// right after the prefix (tree verify: D draft keys at draft_slots).
//
// Cost-balanced ranges: a piece has a fixed cost (q load, the first tile's latency,
// the partial write) worth C = piece_cost keys of the main loop, so each sequence
// is given C virtual keys in front of its real ones (vlen_b = C + len_b, 0 for a
// sequence without keys).  The virtual keys of all sequences are laid end to end
// (T in all) and cut into ranges of
//     q = max(ceil(T / nwy), ceil(max_b len_b / (slots - 1)), min_q)
// keys, range y going to the workgroups of grid row y (one per head group).  A
// range is cut at sequence ends into pieces (its virtual keys are no work), so a
// workgroup whose range starts a second sequence gets C fewer real keys, and every
// workgroup carries about the same cost whatever the length mix.  Sequence b's real
// keys occupy [s_b, s_b + len_b) with s_b = cum_b + C; its pieces come from
// consecutive rows first_b = floor(s_b / q) .. last_b = floor((s_b + len_b - 1) / q),
// the piece of row y writes partial slot y - first_b, and the row holding the last
// piece records the count.  A sequence spans at most floor((len_b - 1) / q) + 2 <=
// slots rows, whatever the device lengths are, so the slots never overflow.  With
// slots == 1 row y takes all of sequence y.  Only host scalars size the grid;
// lengths are read on the device.
struct Piece {
  int b;       // sequence
  int L;       // its prefix length
  int t0, t1;  // key positions [t0, t1) of this piece, inside [lo_b, L_b + D)
  int slot;    // partial slot
  int count;   // on the sequence's last piece, its number of pieces; else 0
};

__device__ __forceinline__ int seq_prefix_len(const FwdParams& P, int b) {
  return max(load_ro(P.prefix_lens, b), 0);
}

__device__ __forceinline__ int seq_lo(const FwdParams& P, int L) {
  return P.window >= 0 ? max(0, L - P.window) : 0;
}

// Keys of sequence b's pieces: its attended prefix and its draft keys (none when it
// has no rows).
__device__ __forceinline__ int seq_len_keys(const FwdParams& P, int b, int L) {
  const int n = seq_rows(P, b);
  return n > 0 ? L - seq_lo(P, L) + (P.draft_slots ? P.draft : n) : 0;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-wide (64-lane) reductions and scan on VALU lane moves instead of LDS permutes:
// DPP inside a 16-lane row (quad xor 1 / xor 2, half-row and row mirror, row shift
// right, broadcast of lanes 15 and 31 into the following rows) and gfx950's row swaps
// across rows.  The control words are the GFX9 DPP encodings.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ int64_t make64(uint32_t lo, uint32_t hi) {
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
// lane moved by DPP control C, rows outside row_mask keep 0, sources outside the row read 0
template <int C, int RowMask = 0xf>
__device__ __forceinline__ int64_t dpp64(int64_t x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(uint64_t)x, C, RowMask, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)x >> 32), C, RowMask, 0xf, true);
  return make64((uint32_t)lo, (uint32_t)hi);
}
template <int C>
__device__ __forceinline__ int dpp32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, C, 0xf, 0xf, true);
}
// sum over all 64 lanes, in every lane
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
  x += dpp64<kDppQuadXor1>(x);
  x += dpp64<kDppQuadXor2>(x);
  x += dpp64<kDppRowHalfMirror>(x);
  x += dpp64<kDppRowMirror>(x);
  // rows 2r and 2r+1, then the two halves: each lane gets both values of the swap
  const uint32_t lo = (uint32_t)(uint64_t)x, hi = (uint32_t)((uint64_t)x >> 32);
  const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  x = make64(a[0], c[0]) + make64(a[1], c[1]);
  const uint32_t lo2 = (uint32_t)(uint64_t)x, hi2 = (uint32_t)((uint64_t)x >> 32);
  const auto d = __builtin_amdgcn_permlane32_swap(lo2, lo2, false, false);
  const auto f = __builtin_amdgcn_permlane32_swap(hi2, hi2, false, false);
  return make64(d[0], f[0]) + make64(d[1], f[1]);
}
// max over all 64 lanes, in every lane
__device__ __forceinline__ int wave_max32(int x) {
  x = max(x, dpp32<kDppQuadXor1>(x));
  x = max(x, dpp32<kDppQuadXor2>(x));
  x = max(x, dpp32<kDppRowHalfMirror>(x));
  x = max(x, dpp32<kDppRowMirror>(x));
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = max((int)a[0], (int)a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return max((int)c[0], (int)c[1]);
}
// inclusive prefix sum over lanes 0..63
__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x) {
  x += dpp64<kDppRowShr1>(x);
  x += dpp64<kDppRowShr2>(x);
  x += dpp64<kDppRowShr4>(x);
  x += dpp64<kDppRowShr8>(x);
  x += dpp64<kDppRowBcast15, 0xa>(x);  // rows 1, 3 add the last lane of rows 0, 2
  x += dpp64<kDppRowBcast31, 0xc>(x);  // rows 2, 3 add lane 31
  return x;
}
__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  return make64(__builtin_amdgcn_readlane((uint32_t)(uint64_t)x, l),
                __builtin_amdgcn_readlane((uint32_t)((uint64_t)x >> 32), l));
}
// a / b for 0 <= a, 0 < b, both wave-uniform: 32-bit division when both fit
__device__ __forceinline__ int64_t udiv64(int64_t a, int64_t b) {
  if ((uint64_t)(a | b) <= 0xffffffffull) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

struct PieceWalk {
  int64_t a, e, q, cum;  // range [a, e) and sequence b's virtual start, in virtual keys
  int b, y, len;
  int Lb;  // sequence b's prefix length when already loaded, else -1 (saves piece() a load)

  __device__ int keys_of(const FwdParams& P, int c) const {
    return seq_len_keys(P, c, seq_prefix_len(P, c));
  }
  __device__ int64_t vlen(const FwdParams& P, int l) const { return l > 0 ? (int64_t)l + P.piece_cost : 0; }

  // Finds row y's first piece.  Returns false when the row has no real keys.  The
  // key counts of the first 64 sequences are loaded once (lane s: sequence s) and
  // serve both passes.
  __device__ bool init(const FwdParams& P, int row) {
    const int lane = threadIdx.x & 63;
    y = row;
    if (P.slots == 1) {
      if (y >= P.batch) return false;
      Lb = seq_prefix_len(P, y);
      if (seq_len_keys(P, y, Lb) == 0) return false;
      b = y;
      q = 0;
      return true;
    }
    const int L0 = lane < P.batch ? seq_prefix_len(P, lane) : 0;
    const int ln0 = lane < P.batch ? seq_len_keys(P, lane, L0) : 0;
    int64_t T = 0;
    int mx = 0;
    for (int c = 0; c < P.batch; c += 64) {
      int l = 0;
      if (c == 0) {
        l = ln0;
      } else if (c + lane < P.batch) {
        l = seq_len_keys(P, c + lane, seq_prefix_len(P, c + lane));
      }
      T += wave_sum64(vlen(P, l));
      mx = max(mx, wave_max32(l));
    }
    T = uniform64(T);
    mx = __builtin_amdgcn_readfirstlane(mx);
    const int nwy = gridDim.y;
    int64_t qq = udiv64(T + nwy - 1, nwy);
    const int64_t qs = udiv64((int64_t)mx + P.slots - 2, P.slots - 1);
    if (qs > qq) qq = qs;
    if (qq < P.min_q) qq = P.min_q;
    q = qq;
    a = (int64_t)y * q;
    if (a >= T) return false;
    e = a + q < T ? a + q : T;
    // the sequence holding virtual key a: inclusive scan over 64 sequences at a time
    int64_t base = 0;
    for (int c = 0; c < P.batch; c += 64) {
      int l = 0;
      if (c == 0) {
        l = ln0;
      } else if (c + lane < P.batch) {
        l = seq_len_keys(P, c + lane, seq_prefix_len(P, c + lane));
      }
      const int64_t vl = vlen(P, l);
      const int64_t incl = wave_incl_scan64(vl);
      const uint64_t hit = __ballot(base + incl > a);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        b = c + f;
        Lb = c == 0 ? __builtin_amdgcn_readlane(L0, f) : -1;
        cum = uniform64(base + readlane64(incl, f) - readlane64(vl, f));
        // a range that ends inside b's virtual keys holds no real key
        return cum + P.piece_cost < e;
      }
      base += readlane64(incl, 63);
    }
    return false;  // unreachable for a < T
  }

  __device__ Piece piece(const FwdParams& P) {
    Piece pc;
    pc.b = __builtin_amdgcn_readfirstlane(b);
    pc.L = __builtin_amdgcn_readfirstlane(Lb >= 0 ? Lb : seq_prefix_len(P, pc.b));
    const int lo = seq_lo(P, pc.L);
    len = seq_len_keys(P, pc.b, pc.L);
    if (P.slots == 1) {
      pc.t0 = lo;
      pc.t1 = lo + len;
      pc.slot = 0;
      pc.count = 1;
      return pc;
    }
    const int64_t sb = cum + P.piece_cost;  // virtual position of b's first real key
    const int64_t s0 = a > sb ? a : sb;
    const int64_t s1 = e < sb + len ? e : sb + len;
    pc.t0 = lo + (int)(s0 - sb);
    pc.t1 = lo + (int)(s1 - sb);
    const int64_t first = udiv64(sb, q), last = udiv64(sb + len - 1, q);
    pc.slot = (int)(y - first);
    pc.count = (y == last) ? (int)(last - first + 1) : 0;
    pc.t0 = __builtin_amdgcn_readfirstlane(pc.t0);
    pc.t1 = __builtin_amdgcn_readfirstlane(pc.t1);
    pc.slot = __builtin_amdgcn_readfirstlane(pc.slot);
    pc.count = __builtin_amdgcn_readfirstlane(pc.count);
    return pc;
  }

  // Advances to the next sequence of the range with real keys in it; false at its end.
  __device__ bool next(const FwdParams& P) {
    if (P.slots == 1) return false;
    cum += vlen(P, len);
    // the next sequence with keys (sequences without rows own none)
    while (cum < e && b + 1 < P.batch) {
      ++b;
      Lb = seq_prefix_len(P, b);
      len = seq_len_keys(P, b, Lb);
      if (len > 0) return cum + P.piece_cost < e;
    }
    return false;
  }
};

// Validates args (host only) and fills the plan.  Returns a VA_ status.  Pointer
// checks (null, alignment) are skipped when check_pointers is false.
int make_plan(const verify_attn_args* a, Plan* plan, bool check_pointers);

// Kernel launchers (one per translation unit).
int launch_block_table(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                       int lg_page, int32_t max_pages, int32_t* block_table, int32_t* kv_lens,
                       hipStream_t stream);
int launch_splitkv_fwd(const verify_attn_args* a, const Plan& p, hipStream_t stream);
// bf16 heads with qk_dim = v_dim = 256: whole-slot-row tiles shared by hpc heads x
// nrg row groups (hpc x nrg in 1x1, 2x1, 4x1, 1x2, 2x2, 1x4); other d is rejected.
int launch_splitkv_tile(const FwdParams& fp, int d, int hpc, int nrg, dim3 grid, hipStream_t stream);
// fp8 MLA heads (qk_dim 576, v_dim 512 = first 512 of the K row), <= 64 rows per head.
int launch_splitkv_mla_fp8(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t stream);
int launch_combine(const verify_attn_args* a, const Plan& p, hipStream_t stream);
int launch_translate_slots(const int32_t* in, int64_t n, const int32_t* full_to_swa, int32_t* out,
                           hipStream_t stream);

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
