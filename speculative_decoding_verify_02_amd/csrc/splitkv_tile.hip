// Split-KV pass for bf16 GQA heads (qk_dim = v_dim = 256) that reads the
// paged cache as whole slot rows.
//
// In the [slot, H_kv, d] layout (the paged view of PR #23146) the K rows of all
// KV heads of one token are adjacent, and a page of P tokens is P * H_kv * d
// contiguous elements.  A workgroup therefore takes HPC KV heads of one
// key range (pieces of sequences) and loads each 16-token block cooperatively: every load
// instruction reads whole runs of a slot row (all HPC heads), so HBM sees long
// contiguous reads instead of one head's 256-byte slices.  Three blocks are in
// flight in registers ahead of the one being computed (the loop is unrolled by
// three so each register set has a fixed name), and each is staged into one of
// two LDS tiles (K and V) one block before it is computed; each wave then reads
// only its own head's slice:
//   QK: A operand = K rows from LDS (ds_read_b128), B = the wave's Q^T rows held
//       in registers, v_mfma_f32_16x16x32_bf16 -> S^T (16 tokens x 16 rows);
//   softmax: online, exp2 domain, row max across the 4 lanes of a row;
//   PV: O^T += V^T P^T with v_mfma_f32_16x16x16_bf16; the V^T operand (4 tokens
//       of one column per lane) comes from one ds_read_b64_tr_b16 per 16
//       columns: in each 16-lane group, lanes 4k..4k+3 address token row k's 16
//       columns and lane c receives column c of the 4 rows; the lane's own 4
//       probabilities are the B operand.
// Waves: HPC heads x NRG row groups (16 rows each).  No merge between waves: each
// wave owns its (head, rows) for the whole piece and writes its partial.

#include <limits.h>
#include <math.h>

#include <type_traits>
#include <utility>

#include "va_internal.h"

namespace va {

namespace {

constexpr int kTB = 16;  // tokens per block
constexpr float kLazy = 8.f;  // log2 headroom of the running max (p <= 256)
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D, int HPC, int NRG>
struct TileGeo {
  static constexpr int W = HPC * NRG;             // waves per workgroup
  static constexpr int RB = D * 2;                // bytes of one head's row
  // LDS row strides, each padded by 32 bytes (rows 8 banks apart): the 16-byte K
  // operand reads (16 rows, 4 lanes per row) and the transposed V reads (8 rows of 32
  // bytes per 32 lanes) then hit distinct banks.  Measured with SQ_LDS_BANK_CONFLICT:
  // 0 conflict cycles, against 20% of the LDS-active cycles with a 16-byte K pad and
  // 77% unpadded
  static constexpr int RSK = HPC * RB + 32;
  static constexpr int RSV = HPC * RB + 32;
  static constexpr int TILEK = kTB * RSK;         // bytes of one K tile
  static constexpr int TILEV = kTB * RSV;         // bytes of one V tile
  static constexpr int CH = HPC * RB / 16;        // 16-byte chunks per token row slice
  static constexpr int NLD = kTB * CH / (64 * W); // loads per thread per block (K; same for V)
  static_assert((kTB * CH) % (64 * W) == 0, "whole loads per thread");
};

}  // namespace

constexpr int kDepth = 3;  // blocks in flight in registers

// f(integral_constant<int, I>) for each I of the sequence, in order: every register
// set of the block ring gets a fixed name in the unrolled loop.
template <class F, int... I>
__device__ __forceinline__ void for_sets(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

template <int D, int HPC, int NRG>
__global__ __launch_bounds__(64 * HPC * NRG) __attribute__((amdgpu_waves_per_eu(1, 1)))
void splitkv_tile_kernel(FwdParams P) {
  using G = TileGeo<D, HPC, NRG>;
  constexpr int KS = D / 32;   // QK k-steps
  constexpr int CT = D / 16;   // O^T column tiles
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][G::TILEK];
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][G::TILEV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;
  const int hc = wave / NRG;          // head within the workgroup
  const int rg = wave % NRG;          // row group of that head
  const int g0 = blockIdx.x * HPC;    // first KV head of the workgroup (HPC divides H_kv)
  const int g = g0 + hc;
  PieceWalk pw;
  if (!pw.init(P, blockIdx.y)) return;  // uniform over the workgroup, before any barrier
  const int row = rg * 16 + n;
  // this thread's load chunks: q = 64*W*u + tid -> token q / CH, head (q % CH) / (RB/16),
  // 16-byte chunk (q % CH) % (RB/16) of that head's row
  const uint32_t k_sslot = (uint32_t)P.k_sslot, v_sslot = (uint32_t)P.v_sslot;
  uint32_t koff[G::NLD], voff[G::NLD];
#pragma unroll
  for (int u = 0; u < G::NLD; ++u) {
    const int c = (64 * G::W * u + tid) % G::CH;
    const int hd = c / (G::RB / 16), cc = c % (G::RB / 16);
    koff[u] = (uint32_t)((g0 + hd) * (uint32_t)P.k_shead + 16 * cc);
    voff[u] = (uint32_t)((g0 + hd) * (uint32_t)P.v_shead + 16 * cc);
  }
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;

  do {
  const Piece pc = pw.piece(P);
  const int b = pc.b;
  const int L = pc.L;
  const int t_begin = pc.t0, t_end = pc.t1;
  const int nblk = (t_end - t_begin + kTB - 1) / kTB;
  const int t_last = t_end - 1;
  if (pc.count > 0 && blockIdx.x == 0 && tid == 0) P.counts[b] = pc.count;

  // the lane's row: draft row_i of sequence b (rows past the sequence's count idle)
  const bool rv = row < P.rows && row / P.group < seq_rows(P, b);
  const int row_i = rv ? row / P.group : 0;
  const bool tree = P.draft_slots != nullptr;
  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;
  // A slot lookup in two parts: lane_raw loads the page id of the lane's token of the
  // block at t0 (its draft slot for tree-verify draft keys) with no branch, and
  // lane_slot turns it into the slot where the value is used, so the wait for the
  // load sits at the use.
  auto lane_raw = [&](int t0) -> int {
    const int t = min(t0 + (lane & (kTB - 1)), t_last);
    const int32_t* src = (tree && t >= L) ? P.draft_slots + b * P.draft + (t - L) : bt_row + (t >> lg);
    // a global (not flat) load: the compiler then waits for it by count and leaves
    // the data loads issued after it in flight
    return *(const __attribute__((address_space(1))) int32_t*)src;
  };
  auto lane_slot = [&](int raw, int t0) -> int {
    const int t = min(t0 + (lane & (kTB - 1)), t_last);
    return (tree && t >= L) ? raw : (raw << lg) | (t & pmask);
  };
  // Page ids: at step b (set s = b % kDepth), pid[s] holds block b + kDepth's and is
  // refilled with block b + 2 kDepth's once used.  A lookup is issued kDepth steps
  // before its use and each register is written and read once per kDepth steps, so
  // the compiler's wait for a lookup leaves the later steps' data loads in flight.
  // The piece's first lookups go out before anything else of its set-up: their round
  // trip overlaps the q loads and row bounds below, and waiting for them never waits
  // for q.
  int first[kDepth], pid[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) first[u] = lane_raw(t_begin + u * kTB);
#pragma unroll
  for (int u = 0; u < kDepth; ++u) pid[u] = lane_raw(t_begin + (kDepth + u) * kTB);
  const uint32_t tbits = (tree && rv) ? tree_bits(P, b, row_i) : 0u;

  // Q^T operands of this wave's 16 rows: k-step ks holds elements 32ks + 8j + [0, 8)
  bf16x8 qB[KS];
  {
    const int hh = rv ? row % P.group : 0;
    const uint8_t* qp = P.q + (int64_t)(seq_row0(P, b) + row_i) * P.q_srow +
                        (int64_t)(g * P.group + hh) * P.q_shead;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (rv) raw = *reinterpret_cast<const u32x4*>(qp + 2 * (32 * ks + 8 * j));
      qB[ks] = as_bf16x8(raw);
    }
  }
  // keys of row i: p - W <= t <= p with p = L + i (prefix and causal draft keys)
  const int row_lo = (P.window >= 0 && rv) ? L + row_i - P.window : INT_MIN;
  const int row_hi = rv ? (tree ? t_last : min(t_last, L + row_i)) : -1;
  // keys every row of the wave sees: blocks inside [wave_lo, wave_hi] need no masking
  // (tree draft keys and capped logits always take the general path)
  int wave_lo = rv ? row_lo : INT_MIN;
  int wave_hi = rv ? (tree ? min(row_hi, L - 1) : row_hi) : INT_MAX;
  if (P.logit_cap > 0.f) wave_hi = INT_MIN;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    wave_lo = max(wave_lo, __shfl_xor(wave_lo, off, 64));
    wave_hi = min(wave_hi, __shfl_xor(wave_hi, off, 64));
  }
  wave_lo = __builtin_amdgcn_readfirstlane(wave_lo);
  wave_hi = __builtin_amdgcn_readfirstlane(wave_hi);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // kDepth register sets: set s holds the blocks b with b % kDepth == s
  u32x4 kr[kDepth][G::NLD], vr[kDepth][G::NLD];
  // Slot s's row starts s * sslot bytes into the cache (the host checks that slot
  // strides and head offsets fit in 32 bits).  When a token row is a whole number of
  // wave loads (CH a multiple of 64), every load instruction of a wave reads one
  // token, so its slot and base address are scalar and the lane adds only its
  // 32-bit offset inside the row.
  auto load_part = [&](auto set, int sl_lane, int u0, int u1) {
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      uint32_t slot;
      if constexpr (G::CH % 64 == 0) {
        slot = __builtin_amdgcn_readlane(sl_lane, (G::W * u + wave) / (G::CH / 64));
      } else {
        slot = __shfl(sl_lane, (64 * G::W * u + tid) / G::CH, 64);
      }
      // read once: non-temporal, so the stream leaves the reused data in the caches
      kr[set][u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(P.k + (uint64_t)slot * k_sslot + koff[u]));
      vr[set][u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(P.v + (uint64_t)slot * v_sslot + voff[u]));
    }
  };
  auto load = [&](auto set, int sl_lane) { load_part(set, sl_lane, 0, G::NLD); };
  // a step issues its block's loads in kParts groups spread over the step, so the
  // CU's vector memory path works while the waves compute
  constexpr int kParts = G::NLD < 4 ? G::NLD : 4;
  auto load_q = [&](auto set, int sl_lane, int part) {
    load_part(set, sl_lane, part * G::NLD / kParts, (part + 1) * G::NLD / kParts);
  };
  auto stage = [&](auto set, int buf) {
#pragma unroll
    for (int u = 0; u < G::NLD; ++u) {
      const int q = 64 * G::W * u + tid;
      const int tok = q / G::CH, c16 = 16 * (q % G::CH);
      *reinterpret_cast<u32x4*>(&kt[buf][tok * G::RSK + c16]) = kr[set][u];
      *reinterpret_cast<u32x4*>(&vt[buf][tok * G::RSV + c16]) = vr[set][u];
    }
  };
  using Sets = std::make_integer_sequence<int, kDepth>;

  {
    for_sets(
        [&](auto set) {
          constexpr int u = decltype(set)::value;
          load(set, lane_slot(first[u], t_begin + u * kTB));
        },
        Sets{});
    stage(std::integral_constant<int, 0>{}, 0);
  }
  __syncthreads();

  const int hoff = hc * G::RB;
  // transposed-read address of this lane inside a V tile: token row 4j + n/4, 4
  // columns starting at 4*(n%4) of each 16-column tile
  const int vlane = (4 * j + (n >> 2)) * G::RSV + hoff + 8 * (n & 3);

  // One block: its set refills with block blk + kDepth, the block is computed from
  // LDS, and block blk + 1 is staged into the other LDS tile.  Steps have no
  // branches, so the compiler keeps exact counts of the loads in flight: blocks past
  // the piece load its last token (a valid address) and are computed with every key
  // masked, which leaves the softmax state unchanged.
  auto step = [&](auto set, int blk) {
    const int buf = blk & 1;
    const int t0 = t_begin + blk * kTB;
    constexpr int si = decltype(set)::value;
    const int sl_next = lane_slot(pid[si], t0 + kDepth * kTB);
    load_q(set, sl_next, 0);

    // a4: S^T = K Q^T for the block's 16 tokens.  All K operand reads go first, then
    // two independent MFMA chains (even and odd k-steps): one LDS round trip and half
    // the accumulator dependence per block, which matters at one wave per SIMD.
    const uint8_t* kp = &kt[buf][n * G::RSK + hoff + 16 * j];
    u32x4 kk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kk[ks] = *reinterpret_cast<const u32x4*>(kp + 64 * ks);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sacc0 = {0.f, 0.f, 0.f, 0.f}, sacc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[ks]), qB[ks], sacc0, 0, 0, 0);
      sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[ks + 1]), qB[ks + 1], sacc1, 0, 0, 0);
    }
    if constexpr (kParts > 1) load_q(set, sl_next, 1);
    const f32x4 sacc = sacc0 + sacc1;

    // online softmax: lane holds row n's scores for tokens 4j + r
    float sc[4];
    if (t0 >= wave_lo && t0 + (kTB - 1) <= wave_hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = sacc[r] * P.c_log2;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * j + r;
        const bool ok = key_ok(t, row_lo, row_hi, L, tbits, tree);
        sc[r] = ok ? sacc[r] * P.c_log2 : -INFINITY;
      }
      if (P.logit_cap > 0.f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = sc[r] == -INFINITY ? sc[r] : cap_log2(sc[r], P.logit_cap);
      }
    }
    const float bmax = rows4_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    // the reference max moves only when a score passes it by more than kLazy, so
    // most blocks leave the accumulator alone; p = 2^(s - m) stays <= 2^kLazy
    const bool grow = bmax > m_run + kLazy;
    const float m_new = grow ? bmax : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = __builtin_amdgcn_exp2f(sc[r] - m_use);
      psum += sc[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(grow)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) oacc[ct] *= alpha;
    }
    const __bf16 p0 = (__bf16)sc[0], p1 = (__bf16)sc[1], p2 = (__bf16)sc[2], p3 = (__bf16)sc[3];
    const s16x4 pB = {__builtin_bit_cast(short, p0), __builtin_bit_cast(short, p1),
                      __builtin_bit_cast(short, p2), __builtin_bit_cast(short, p3)};

    if constexpr (kParts > 2) load_q(set, sl_next, 2);
    // a5: O^T += V^T P^T, V^T from transposed LDS reads
    __attribute__((address_space(3))) char* vb =
        (__attribute__((address_space(3))) char*)vt[buf] + vlane;
    // all transposed reads first, then the MFMAs (one LDS round trip per block)
    i16x4 va[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      va[ct] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(vb + 32 * ct));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[ct], pB, oacc[ct], 0, 0, 0);

    if constexpr (kParts > 3) load_q(set, sl_next, 3);
    pid[si] = lane_raw(t0 + 2 * kDepth * kTB);
    stage(std::integral_constant<int, (decltype(set)::value + 1) % kDepth>{}, buf ^ 1);
    __syncthreads();
  };
  for (int blk = 0; blk < nblk; blk += kDepth)
    for_sets([&](auto set) { step(set, blk + decltype(set)::value); }, Sets{});

  // each lane summed only its own tokens: total the 4 lanes of the row
  l_run = rows4_sum(l_run);
  if (rv) {
    const int64_t split_id = ((int64_t)b * P.hkv + g) * P.slots + pc.slot;
    const float inv = l_run > 0.f ? P.v_scale / l_run : 0.f;
    // lane holds O[row][16ct + 4j + r], r = 0..3
    float* po = P.part_o + (split_id * P.rows + row) * D + 4 * j;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 o = oacc[ct];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= inv;
      *reinterpret_cast<f32x4*>(po + 16 * ct) = o;
    }
    if (j == 0)
      P.part_lse[split_id * P.rows + row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
  } while (pw.next(P));
}

// d = 256 only (d = 128 streams better through the generic kernel); at most 4 waves
int launch_splitkv_tile(const FwdParams& fp, int d, int hpc, int nrg, dim3 grid, hipStream_t st) {
  if (d != 256) return VA_EUNSUPPORTED;
#define VA_TILE(H_, R_)                                                                        \
  return launch_kernel(reinterpret_cast<const void*>(&splitkv_tile_kernel<256, H_, R_>), grid, \
                       dim3(64 * (H_) * (R_)), fp, st)
  switch (hpc * 10 + nrg) {
    case 11: VA_TILE(1, 1);
    case 21: VA_TILE(2, 1);
    case 41: VA_TILE(4, 1);
    case 12: VA_TILE(1, 2);
    case 22: VA_TILE(2, 2);
    case 14: VA_TILE(1, 4);
    default: return VA_EUNSUPPORTED;
  }
#undef VA_TILE
}

}  // namespace va
