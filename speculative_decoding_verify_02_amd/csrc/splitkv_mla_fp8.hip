// Split-KV pass for an fp8 MLA head: one shared latent KV head whose cached row is
// qk_dim = 576 e4m3fn bytes, with V the first v_dim = 512 bytes of the same row
// (PR #23146 review: qk_head_dim differs from v_head_dim; V is read from the K
// cache view).  The dense M dimension is G*D <= 64 query rows (16 heads x 4 drafts
// on one GPU's share), so each token costs ~140 kflop: this kernel is built to keep
// the MFMA pipes busy while streaming the cache.
//
//   workgroup = (KV head g, key range y: pieces of sequences), 4 waves; wave w owns rows
//   16w .. 16w+15.  Blocks of 128 tokens: the workgroup loads a block's K rows
//   coalesced into registers (the next block's loads are in flight while the
//   current block computes), stages them in one shared LDS tile, and every wave
//   reads its operands from there.
//   QK: S^T = K Q^T.  For d < 512 with v_mfma_f32_16x16x128_f8f6f4: K bytes as
//       they are, and the bf16 q as two e4m3 terms hi + lo/16 (the lo product is
//       scaled by 2^-4 through the MFMA's MX block scale), ~2^-9 relative error in
//       q, the precision bf16 itself carries.  The rope tail d in [512, 576) uses
//       v_mfma_f32_16x16x32_bf16 with K widened exactly to bf16 (every e4m3fn value
//       is a bf16 value) and q in bf16.
//   softmax: online, exp2 domain, row max across the 4 lanes of a row.
//   PV: O^T += V^T P^T with v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3).  P enters
//       as two e4m3 terms, hi = e4m3(256 p) and lo = e4m3(16 (256 p - hi)) with the
//       lo product scaled by 2^-4 through the MFMA's MX block scale: about 8
//       significant bits per probability, close to bf16.  p <= 1, so 256 p never
//       overflows, and the factor keeps small probabilities out of the subnormal
//       range; it is divided out at the end.  The running sum l uses the
//       unrounded fp32 p.  The A operand (32 tokens
//       of one V column per lane) comes from four ds_read_b64_tr_b8 transposed LDS
//       reads: in each 16-lane group, lanes 2k and 2k+1 address the two 8-byte
//       halves of a 16-column slice of token row k, and lane c receives column c of
//       the 8 rows.

#include <limits.h>
#include <math.h>

#include "va_internal.h"

namespace va {

namespace {

constexpr int kMB = 128;              // tokens per block
constexpr int kKRB = 576;             // K row bytes
constexpr int kVRB = 512;             // V bytes per row (first part of the K row)
constexpr int kRS = kKRB + 16;        // LDS row stride: 16-lane operand reads hit distinct banks
constexpr int kNCH = kKRB / 16;       // 16-byte chunks per row
constexpr int kNLD = kMB * kNCH / 256;  // coalesced loads per thread per block
constexpr int kCT = kVRB / 16;        // O^T column tiles
constexpr int kQRS = 2 * kKRB + 16;  // LDS row stride of a wave's bf16 Q rows
constexpr float kPScale = 256.f;
constexpr int kE8M0One = 127;         // MX block scale exponents (bias 127)
constexpr int kE8M0Sixteenth = 123;
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

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

// Slots of the block's tokens t0 + lane and t0 + 64 + lane (clamped to the piece).
__device__ __forceinline__ void block_slots(const int32_t* bt_row, int t0, int t_last, int lane,
                                            int lg, int pmask, int& sa, int& sb) {
  const int ta = min(t0 + lane, t_last), tb = min(t0 + 64 + lane, t_last);
  sa = (bt_row[ta >> lg] << lg) | (ta & pmask);
  sb = (bt_row[tb >> lg] << lg) | (tb & pmask);
}

// Token of score slot i (0..31) of lane group j: tile i/4, accumulator row 4j + i%4.
__device__ __forceinline__ int slot_token(int j, int i) { return 16 * (i >> 2) + 4 * j + (i & 3); }

// LDS of the one workgroup a compute unit holds: the shared K tile and each wave's
// staged Q rows.
__shared__ __attribute__((aligned(16))) uint8_t s_tile[kMB * kRS];
__shared__ __attribute__((aligned(16))) uint8_t s_qtile[kWaves][16 * kQRS];

// One piece: keys [pc.t0, pc.t1) of sequence pc.b for KV head g -> partial slot
// pc.slot.  Kept out of line so the piece loop adds no register pressure to it.
__device__ __noinline__ void mla_piece(const FwdParams& P, const Piece pc, int g) {
  uint8_t* tile = s_tile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int row = wave * 16 + n;
  const bool rv = row < P.rows;
  const int row_i = rv ? row / P.group : 0;  // draft index of this lane's row
  uint8_t* qw = s_qtile[wave];
  const uint8_t* kg = P.k + (int64_t)g * P.k_shead;
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;
  const int b = pc.b;
  const int L = pc.L;
  const int t_begin = pc.t0, t_end = pc.t1;
  const int nblk = (t_end - t_begin + kMB - 1) / kMB;
  const int t_last = t_end - 1;
  if (pc.count > 0 && g == 0 && tid == 0) P.counts[b] = pc.count;

  // this wave's 16 Q rows go to its own LDS rows: for d < 512 as two e4m3 terms
  // (hi = e4m3(q), lo = e4m3(16 (q - hi)), together ~2^-9 relative error, the
  // precision of the bf16 q itself) for the fp8 MFMA, and the 64-wide rope tail
  // d >= 512 as bf16.  Row layout: hi[512] | lo[512] | bf16 tail[64].
  {
#pragma unroll
    for (int c = 0; c < 16 * (kVRB / 8) / 64; ++c) {       // 16 chunks of 8 values per lane
      const int q = 64 * c + lane;
      const int r = q / (kVRB / 8), ch = q % (kVRB / 8);
      const int qrow = wave * 16 + r;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < P.rows) {
        const int i = qrow / P.group, hh = qrow % P.group;
        raw = *reinterpret_cast<const u32x4*>(P.q + (int64_t)(b * P.draft + i) * P.q_srow +
                                              (int64_t)(g * P.group + hh) * P.q_shead + 16 * ch);
      }
      float x[8];  // q elements, saturated to the e4m3 range (+-448)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = fminf(fmaxf(__uint_as_float(raw[e] << 16), -448.f), 448.f);
        x[2 * e + 1] = fminf(fmaxf(__uint_as_float(raw[e] & 0xffff0000u), -448.f), 448.f);
      }
      uint32_t hi[2], lo[2];
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
        hi[h] = (uint32_t)w;
        lo[h] = (uint32_t)wl;
      }
      *reinterpret_cast<u32x2*>(qw + r * kQRS + 8 * ch) = u32x2{hi[0], hi[1]};
      *reinterpret_cast<u32x2*>(qw + r * kQRS + kVRB + 8 * ch) = u32x2{lo[0], lo[1]};
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {                             // 16 rows x 8 tail chunks
      const int q = 64 * c + lane;
      const int r = q / 8, ch = q % 8;
      const int qrow = wave * 16 + r;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < P.rows) {
        const int i = qrow / P.group, hh = qrow % P.group;
        raw = *reinterpret_cast<const u32x4*>(P.q + (int64_t)(b * P.draft + i) * P.q_srow +
                                              (int64_t)(g * P.group + hh) * P.q_shead +
                                              2 * kVRB + 16 * ch);
      }
      *reinterpret_cast<u32x4*>(qw + r * kQRS + 2 * kVRB + 16 * ch) = raw;
    }
  }
  // keys of row i: p - W <= t <= p with p = L + i (prefix and causal draft keys)
  const int row_lo = (P.window >= 0 && rv) ? L + row_i - P.window : INT_MIN;
  const int row_hi = rv ? min(t_last, L + row_i) : -1;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[kCT];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;

  // coalesced block load: thread chunk q = 256u + tid -> token q / 36, chunk q % 36
  u32x4 kreg[kNLD];
  auto load = [&](int sa, int sb) {
#pragma unroll
    for (int u = 0; u < kNLD; ++u) {
      const int q = 256 * u + tid;
      const int tok = q / kNCH;
      const int xa = __shfl(sa, tok & 63, 64), xb = __shfl(sb, tok & 63, 64);
      const int sl = tok < 64 ? xa : xb;
      kreg[u] = *reinterpret_cast<const u32x4*>(kg + (int64_t)sl * P.k_sslot + 16 * (q % kNCH));
    }
  };
  int sa, sb, na = 0, nb = 0;
  block_slots(bt_row, t_begin, t_last, lane, lg, pmask, sa, sb);
  load(sa, sb);
  if (nblk > 1) block_slots(bt_row, t_begin + kMB, t_last, lane, lg, pmask, na, nb);

  for (int blk = 0; blk < nblk; ++blk) {
    const int t0 = t_begin + blk * kMB;
    __syncthreads();  // every wave is done reading the previous block's tile
#pragma unroll
    for (int u = 0; u < kNLD; ++u) {
      const int q = 256 * u + tid;
      *reinterpret_cast<u32x4*>(tile + (q / kNCH) * kRS + 16 * (q % kNCH)) = kreg[u];
    }
    __syncthreads();
    if (blk + 1 < nblk) {
      load(na, nb);  // next block in flight during this block's math
      if (blk + 2 < nblk) block_slots(bt_row, t0 + 2 * kMB, t_last, lane, lg, pmask, na, nb);
    }

    // a4: S^T for 8 token tiles
    f32x4 sacc[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // d < 512: fp8 x fp8 (K bytes as they are, q as hi + lo terms); lane group j
    // holds elements 128kb + 32j + [0, 32) of its token (A) and of its row (B)
#pragma unroll
    for (int kb = 0; kb < kVRB / 128; ++kb) {
      const uint8_t* qp = qw + n * kQRS + 128 * kb + 32 * j;
      const u32x4 h0 = *reinterpret_cast<const u32x4*>(qp);
      const u32x4 h1 = *reinterpret_cast<const u32x4*>(qp + 16);
      const u32x4 l0 = *reinterpret_cast<const u32x4*>(qp + kVRB);
      const u32x4 l1 = *reinterpret_cast<const u32x4*>(qp + kVRB + 16);
      const i32x8 qh = __builtin_bit_cast(i32x8, u32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
      const i32x8 ql = __builtin_bit_cast(i32x8, u32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]});
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint8_t* kp = tile + (16 * tt + n) * kRS + 128 * kb + 32 * j;
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(kp);
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(kp + 16);
        const i32x8 ka = __builtin_bit_cast(i32x8, u32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]});
        sacc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qh, sacc[tt], 0, 0, 0, 0, 0, 0);
        sacc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, ql, sacc[tt], 0, 0, 0,
                                                                    kE8M0One, 0, kE8M0Sixteenth);
      }
    }
    // rope tail d in [512, 576): bf16 k-steps, lane group j holds 512 + 32h + 8j + [0, 8)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 qr = *reinterpret_cast<const u32x4*>(qw + n * kQRS + 2 * kVRB + 2 * (32 * h + 8 * j));
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const u32x2 kr = *reinterpret_cast<const u32x2*>(tile + (16 * tt + n) * kRS + kVRB + 32 * h + 8 * j);
        const u32x2 w0 = fp8x4_to_bf16x4(kr[0]), w1 = fp8x4_to_bf16x4(kr[1]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]}), as_bf16x8(qr), sacc[tt], 0, 0, 0);
      }
    }

    // online softmax over the lane's 32 scores (row n)
    float sc[32];
    float bmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int t = t0 + slot_token(j, e);
      const bool ok = (t >= row_lo) && (t <= row_hi);
      const float v = ok ? sacc[e >> 2][e & 3] * P.c_log2 : -INFINITY;
      sc[e] = v;
      bmax = fmaxf(bmax, v);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += sc[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // the accumulator lives in AGPRs: rescale only when some row's max moved
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) oacc[ct] *= alpha;
    }
    // P in two e4m3 terms: hi = e4m3(256 p), lo = e4m3(16 (256 p - hi)); the lo
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
    for (int r = 0; r < 4; ++r) voff[r] = slot_token(j, 8 * r + (n >> 1)) * kRS + 8 * (n & 1);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      i32x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            reinterpret_cast<lds_i32x2*>(lbase + voff[r] + 16 * ct));
        a[2 * r] = x[0];
        a[2 * r + 1] = x[1];
      }
      oacc[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, pb, oacc[ct], 0, 0, 0, 0, 0, 0);
      oacc[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, pl, oacc[ct], 0, 0, 0, kE8M0One,
                                                                  0, kE8M0Sixteenth);
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
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void splitkv_mla_fp8_kernel(FwdParams P) {
  PieceWalk pw;
  if (!pw.init(P, blockIdx.y)) return;  // uniform over the workgroup, before any barrier
  do {
    mla_piece(P, pw.piece(P), blockIdx.x);
  } while (pw.next(P));
}

int launch_splitkv_mla_fp8(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t st) {
  if (p.rows > 64) return VA_EUNSUPPORTED;
  return launch_kernel(reinterpret_cast<const void*>(&splitkv_mla_fp8_kernel), grid, dim3(256),
                       fp, st);
}

}  // namespace va
