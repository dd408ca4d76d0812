// Split-KV pass for an fp8 MLA head: one shared latent KV head whose cached row is
// qk_dim = 576 e4m3fn bytes, with V the first v_dim = 512 bytes of the same row
// (PR #23146 review: qk_head_dim differs from v_head_dim; V is read from the K
// cache view).  The dense M dimension is G*D <= 64 query rows (16 heads x 4 drafts
// on one GPU's share), so each key costs ~140 kflop: the kernel keeps the MFMA
// pipes fed from LDS while the cache streams in behind them.
//
//   workgroup = (KV head g, key range y: pieces of sequences), 4 waves; wave w owns
//   rows 16w .. 16w+15 and keeps their q in registers for the whole piece.
//   Tiles of 128 keys stream into a two-tile LDS ring with global_load_lds_dwordx4
//   (one wave instruction copies one key's 576-byte row, 36 lanes x 16 bytes), so
//   no registers hold data in flight: the next tile lands while this one computes.
//   Page ids travel the same way (global_load_lds_dword), so the vector-memory
//   counter covers everything a wave waits for and one vmcnt(0) per tile suffices.
//   LDS rows sit at 592 t + 32 (t / 16) bytes: the 16 rows of an MFMA operand read
//   and the 8 rows of a transposed read all fall on distinct banks.
//   QK: S^T = K Q^T.  For d < 512 with v_mfma_f32_16x16x128_f8f6f4: K bytes as
//       they are, and the bf16 q as two e4m3 terms hi + lo/16 (the lo product is
//       scaled by 2^-4 through the MFMA's MX block scale), ~2^-9 relative error in
//       q, the precision bf16 itself carries.  The rope tail d in [512, 576) uses
//       v_mfma_f32_16x16x32_bf16 with K widened exactly to bf16 (every e4m3fn value
//       is a bf16 value) and q in bf16.
//   softmax: online, exp2 domain, row max across the 4 lanes of a row.  The
//       reference max moves only when a score passes it by more than one (log2
//       units), so p <= 2 and most tiles skip rescaling the accumulator.
//   PV: O^T += V^T P^T with v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3).  P enters
//       as two e4m3 terms, hi = e4m3(128 p) and lo = e4m3(16 (128 p - hi)) with the
//       lo product scaled by 2^-4 through the MFMA's MX block scale: about 8
//       significant bits per probability, close to bf16.  128 p <= 256 never
//       overflows e4m3, and the factor keeps small probabilities out of the
//       subnormal range; it is divided out at the end.  The running sum l uses the
//       unrounded fp32 p.  The A operand (32 keys of one V column per lane) comes
//       from four ds_read_b64_tr_b8 transposed LDS reads: in each 16-lane group,
//       lanes 2k and 2k+1 address the two 8-byte halves of a 16-column slice of key
//       row k, and lane c receives column c of the 8 rows.

#include <limits.h>
#include <math.h>

#include "va_internal.h"

namespace va {

namespace {

constexpr int kMB = 128;              // keys per tile
constexpr int kKRB = 576;             // K row bytes
constexpr int kVRB = 512;             // V bytes per row (first part of the K row)
constexpr int kRS = kKRB + 16;        // LDS row stride
constexpr int kTileBytes = 76032;     // row_off(127) + 576, rounded up to 128
constexpr int kCT = kVRB / 16;        // O^T column tiles
constexpr int kKPW = kMB / kWaves;    // keys each wave copies per tile
constexpr float kPScale = 128.f;      // P scale for e4m3 (p <= 2^kLazy, so 128 p <= 256 < 448)
constexpr float kLazy = 1.f;          // log2 headroom before the running max is moved
constexpr int kE8M0One = 127;         // MX block scale exponents (bias 127)
constexpr int kE8M0Sixteenth = 123;
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Byte offset of key row t inside a tile.  The 16-byte slot of row t mod 16 is
// 5 t + 2 (t / 16): distinct for the 16 consecutive rows of an operand read and for
// the rows {4j + i, 16 + 4j + i} (i < 4) a transposed read takes together.
__device__ __forceinline__ int row_off(int t) { return t * kRS + (t >> 4) * 32; }
static_assert(127 * kRS + 7 * 32 + kKRB <= kTileBytes, "tile holds 128 rows");

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t x) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Copies to LDS at `lds` + lane * size straight from global memory.  Inline assembly,
// so the compiler (which does not see these copies) adds no waits of its own before
// LDS reads; the waits are explicit.  M0 holds the wave's LDS base and needs one
// wait state before the copy reads it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
// Same with a wave-uniform base in SGPRs and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Token of score slot i (0..31) of lane group j: tile i/4, accumulator row 4j + i%4.
__device__ __forceinline__ int slot_token(int j, int i) { return 16 * (i >> 2) + 4 * j + (i & 3); }

// LDS of the one workgroup a compute unit holds: the two-tile ring and each wave's
// page ids for its keys of the next two tiles.
__shared__ __attribute__((aligned(128))) uint8_t s_ring[2][kTileBytes];
__shared__ __attribute__((aligned(16))) int32_t s_pid[2][kWaves][kKPW];

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void splitkv_mla_fp8_kernel(FwdParams P) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.x;
  PieceWalk pw;
  if (!pw.init(P, blockIdx.y)) return;  // uniform over the workgroup, before any barrier

  const int row = wave * 16 + n;
  const bool tree = P.draft_slots != nullptr;
  const uint8_t* kg = P.k + (int64_t)g * P.k_shead;
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;

  do {
  const Piece pc = pw.piece(P);
  const int b = pc.b;
  const int L = pc.L;
  const int t_begin = pc.t0, t_end = pc.t1;
  const int ntile = (t_end - t_begin + kMB - 1) / kMB;
  const int t_last = t_end - 1;
  if (pc.count > 0 && g == 0 && tid == 0) P.counts[b] = pc.count;
  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;
  // the lane's row: draft row_i of sequence b (rows past the sequence's count idle)
  const bool rv = row < P.rows && row / P.group < seq_rows(P, b);
  const int row_i = rv ? row / P.group : 0;

  // page ids of this wave's keys of tile k -> s_pid[k % 2][wave]: entry e is the
  // page of the wave's first key plus e, clamped to the table row
  auto copy_pids = [&](int k) {
    const int tw = min(t_begin + k * kMB + wave * kKPW, t_last);
    const int e = min((tw >> lg) + lane, P.max_pages - 1);
    if (lane < kKPW) dma4(bt_row + e, lds_addr(&s_pid[k & 1][wave][0]));
  };
  // this wave's keys of tile k -> ring buffer k % 2 (one key row per instruction).
  // Lane l < 32 looks up the slot of key l with one LDS read; each copy then takes
  // its key's slot from that lane into a scalar base address.
  auto copy_tile = [&](int k) {
    const int t0 = t_begin + k * kMB + wave * kKPW;
    const int pbase = min(t0, t_last) >> lg;
    uint8_t* ring = s_ring[k & 1];
    const int tl = min(t0 + (lane & (kKPW - 1)), t_last);
    int slot_l = (s_pid[k & 1][wave][(tl >> lg) - pbase] << lg) | (tl & pmask);
    if (tree && t0 + kKPW - 1 >= L)   // tree verify: draft keys at their own slots
      slot_l = tl >= L ? P.draft_slots[b * P.draft + (tl - L)] : slot_l;
#pragma unroll
    for (int u = 0; u < kKPW; ++u) {
      const int slot = __builtin_amdgcn_readlane(slot_l, u);
      if (lane < kKRB / 16)
        dma16_s(kg + (int64_t)slot * P.k_sslot, 16 * lane, lds_addr(ring + row_off(wave * kKPW + u)));
    }
  };

  copy_pids(0);
  if (ntile > 1) copy_pids(1);
  wait_copies();
  copy_tile(0);

  // this wave's 16 q rows in registers: for d < 512 as two e4m3 terms (hi = e4m3(q),
  // lo = e4m3(16 (q - hi)), together ~2^-9 relative error, the precision of the
  // bf16 q itself), the 64-wide rope tail d >= 512 as bf16.  Lane group j holds
  // elements 128kb + 32j + [0, 32) (and 512 + 32h + 8j + [0, 8) of the tail), the
  // k-slots of the K operand read below.
  i32x8 qh[kVRB / 128], ql[kVRB / 128];
  u32x4 qr[2];
  {
    const int hh = rv ? row % P.group : 0;
    const uint8_t* qp =
        P.q + (int64_t)(seq_row0(P, b) + row_i) * P.q_srow + (int64_t)(g * P.group + hh) * P.q_shead;
#pragma unroll
    for (int kb = 0; kb < kVRB / 128; ++kb) {
      u32x4 raw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        raw[c] = rv ? *reinterpret_cast<const u32x4*>(qp + 2 * (128 * kb + 32 * j + 8 * c))
                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[8];  // q elements, saturated to the e4m3 range (+-448)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = fminf(fmaxf(__uint_as_float(raw[c][e] << 16), -448.f), 448.f);
          x[2 * e + 1] = fminf(fmaxf(__uint_as_float(raw[c][e] & 0xffff0000u), -448.f), 448.f);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h], x[4 * h + 1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h + 2], x[4 * h + 3], w, true);
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          const f32x2 c2 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
          int wl = __builtin_amdgcn_cvt_pk_fp8_f32((x[4 * h] - a[0]) * 16.f,
                                                   (x[4 * h + 1] - a[1]) * 16.f, 0, false);
          wl = __builtin_amdgcn_cvt_pk_fp8_f32((x[4 * h + 2] - c2[0]) * 16.f,
                                               (x[4 * h + 3] - c2[1]) * 16.f, wl, true);
          qh[kb][2 * c + h] = w;
          ql[kb][2 * c + h] = wl;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      qr[h] = rv ? *reinterpret_cast<const u32x4*>(qp + 2 * (kVRB + 32 * h + 8 * j))
                 : u32x4{0u, 0u, 0u, 0u};
  }
  // keys of row i: p - W <= t <= p with p = L + i (prefix and causal draft keys)
  const int row_lo = (P.window >= 0 && rv) ? L + row_i - P.window : INT_MIN;
  const int row_hi = rv ? (tree ? t_last : min(t_last, L + row_i)) : -1;
  const uint32_t tbits = (tree && rv) ? tree_bits(P, b, row_i) : 0u;
  // keys every row of the wave sees: tiles inside [wave_lo, wave_hi] need no masking
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
  f32x4 oacc[kCT];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < ntile; ++k) {
    // this wave's copies of tile k (and page ids of tile k + 1) have landed; the
    // barrier shows every wave's and frees the buffer tile k - 1 was computed from
    wait_copies();
    __syncthreads();
    if (k + 1 < ntile) copy_tile(k + 1);
    if (k + 2 < ntile) copy_pids(k + 2);

    const int t0 = t_begin + k * kMB;
    const uint8_t* tile = s_ring[k & 1];

    // a4: S^T for 8 token tiles
    f32x4 sacc[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // d < 512: fp8 x fp8 (K bytes as they are, q as hi + lo terms).  Token tiles go
    // in pairs so the two products into one accumulator are not back to back.
#pragma unroll
    for (int kb = 0; kb < kVRB / 128; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 8; tt += 2) {
        i32x8 ka[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint8_t* kp = tile + row_off(16 * (tt + e) + n) + 128 * kb + 32 * j;
          const u32x4 k0 = *reinterpret_cast<const u32x4*>(kp);
          const u32x4 k1 = *reinterpret_cast<const u32x4*>(kp + 16);
          ka[e] = __builtin_bit_cast(i32x8, u32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]});
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
          sacc[tt + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[e], qh[kb], sacc[tt + e], 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 2; ++e)
          sacc[tt + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[e], ql[kb], sacc[tt + e], 0, 0, 0,
                                                                          kE8M0One, 0, kE8M0Sixteenth);
      }
    }
    // rope tail d in [512, 576): bf16 k-steps, lane group j holds 512 + 32h + 8j + [0, 8)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const u32x2 kr = *reinterpret_cast<const u32x2*>(tile + row_off(16 * tt + n) + kVRB + 32 * h + 8 * j);
        const u32x2 w0 = fp8x4_to_bf16x4(kr[0]), w1 = fp8x4_to_bf16x4(kr[1]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]}), as_bf16x8(qr[h]), sacc[tt], 0, 0, 0);
      }
    }

    // online softmax over the lane's 32 scores (row n)
    float sc[32];
    float bmax = -INFINITY;
    if (t0 >= wave_lo && t0 + kMB - 1 <= wave_hi) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        sc[e] = sacc[e >> 2][e & 3] * P.c_log2;
        bmax = fmaxf(bmax, sc[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int t = t0 + slot_token(j, e);
        const bool ok = key_ok(t, row_lo, row_hi, L, tbits, tree);
        sc[e] = ok ? sacc[e >> 2][e & 3] * P.c_log2 : -INFINITY;
      }
      if (P.logit_cap > 0.f) {
#pragma unroll
        for (int e = 0; e < 32; ++e) sc[e] = sc[e] == -INFINITY ? sc[e] : cap_log2(sc[e], P.logit_cap);
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) bmax = fmaxf(bmax, sc[e]);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    // the reference max moves only when a score passes it by more than kLazy, so
    // most tiles leave the accumulator alone; p = 2^(s - m) stays <= 2^kLazy
    const bool grow = bmax > m_run + kLazy;
    const float m_new = grow ? bmax : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += sc[e];
    }
    // the accumulator lives in AGPRs: rescale only when some row with a nonzero
    // accumulator moved its max
    if (__any(grow && m_run != -INFINITY)) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) oacc[ct] *= alpha;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P in two e4m3 terms: hi = e4m3(128 p), lo = e4m3(16 (128 p - hi)); the lo
    // product enters the same accumulator through the MFMA's B scale 2^-4.  The
    // pair keeps about 8 significant bits of each probability.
    i32x8 pb, pl;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const float x0 = sc[4 * d] * kPScale, x1 = sc[4 * d + 1] * kPScale;
      const float x2 = sc[4 * d + 2] * kPScale, x3 = sc[4 * d + 3] * kPScale;
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
      pb[d] = w;
      const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      int wl = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - h01[0]) * 16.f, (x1 - h01[1]) * 16.f, 0, false);
      wl = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - h23[0]) * 16.f, (x3 - h23[1]) * 16.f, wl, true);
      pl[d] = wl;
    }

    // a5: O^T += V^T P^T, V^T via transposed LDS reads (tokens of slots 8r..8r+7)
    __attribute__((address_space(3))) char* lbase = (__attribute__((address_space(3))) char*)tile;
    int voff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) voff[r] = row_off(slot_token(j, 8 * r + (n >> 1))) + 8 * (n & 1);
#pragma unroll
    for (int ct = 0; ct < kCT; ct += 2) {
      i32x8 a[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              reinterpret_cast<lds_i32x2*>(lbase + voff[r] + 16 * (ct + e)));
          a[e][2 * r] = x[0];
          a[e][2 * r + 1] = x[1];
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
        oacc[ct + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[e], pb, oacc[ct + e], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        oacc[ct + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[e], pl, oacc[ct + e], 0, 0, 0,
                                                                        kE8M0One, 0, kE8M0Sixteenth);
    }
  }

  // each lane summed only its own tokens: total the 4 lanes of the row
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (rv) {
    const int64_t split_id = ((int64_t)b * P.hkv + g) * P.slots + pc.slot;
    const float inv = l_run > 0.f ? P.v_scale / (l_run * kPScale) : 0.f;
    float* po = P.part_o + (split_id * P.rows + row) * kVRB + 4 * j;
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      f32x4 o = oacc[ct];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= inv;
      *reinterpret_cast<f32x4*>(po + 16 * ct) = o;
    }
    if (j == 0)
      P.part_lse[split_id * P.rows + row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
  __syncthreads();  // every wave is done with the ring before the next piece refills it
  } while (pw.next(P));
}

int launch_splitkv_mla_fp8(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t st) {
  if (p.rows > 64) return VA_EUNSUPPORTED;
  return launch_kernel(reinterpret_cast<const void*>(&splitkv_mla_fp8_kernel), grid, dim3(256),
                       fp, st);
}

}  // namespace va
