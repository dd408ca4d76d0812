// Split-KV pass for an fp8 MLA head: one shared latent KV head whose cached row is
// qk_dim = 576 e4m3fn bytes, with V the first v_dim = 512 bytes of the same row
// (PR #23146 review: qk_head_dim differs from v_head_dim; V is read from the K
// cache view).  The dense M dimension is G*D <= 64 query rows (16 heads x 4 drafts
// on one GPU's share), so each key costs ~140 kflop and the kernel is built to keep
// the matrix cores fed while the cache streams into LDS behind them.
//
//   workgroup = (KV head g, key range y: pieces of sequences), 8 waves, two per
//   SIMD.  Wave w = (row group rg = w % 4, half hf = w / 4): the pair (rg, 0),
//   (rg, 1) shares query rows 16 rg .. 16 rg + 15, whose q both keep in registers
//   (each loads and converts half of it and hands that half to the other).
//   Per tile of 128 keys:
//     QK  wave hf scores keys 64 hf .. 64 hf + 63 of the tile (S^T = K Q^T);
//     the pair swaps row maxima through LDS, so both take the same running max,
//     then swaps its probabilities (two e4m3 bytes each), so both hold P for all
//     128 keys;
//     PV  wave hf accumulates output columns 256 hf .. 256 hf + 255 over all 128
//     keys (O^T += V^T P^T).
//   Two waves per SIMD let one wave's softmax, exchanges and waits run under the
//   other's matrix instructions; each wave holds 16 rows x 256 fp32 columns.
//
// Memory: the 512 latent bytes of each key stream into a two-tile LDS ring with
// global_load_lds_dwordx4, one 64-lane instruction per two keys (1 KB), so no
// registers hold data in flight.  A wave's 8 copies of the next tile are spread over
// its QK phase, so a copy that waits for room in the memory queue stalls the wave
// between matrix instructions rather than before them.  The 64 rope bytes, read only
// by QK, go to a single rope buffer that is refilled for the next tile once every
// wave has passed the max exchange.  One vmcnt(0) per tile is the only wait for
// copies; the copies are inline assembly, so the compiler adds none of its own, and
// every compiler-visible load of a tile is issued before its copies.
//   Latent row t sits at 512 t with 16-byte chunk c stored at chunk c ^ f(t),
//   f(t) = (t % 16) ^ 8 ((t / 16) % 2): the 16 rows of an operand read and the 16
//   rows {0..7, 16..23} (or {8..15, 24..31}) of a transposed read fall on distinct
//   banks.  Rope row t sits at 64 t with chunk c stored at c ^ ((t / 4) % 4).
//
//   QK: for d < 512 v_mfma_f32_16x16x128_f8f6f4 with the K bytes as they are and
//       the bf16 q, scaled per row into [128, 256) by a power of two, as two e4m3
//       terms hi + lo (~2^-9 of the row's largest magnitude, the precision bf16
//       itself carries, for any finite q); the scores take the power of two back
//       with sm_scale.  The rope tail d in
//       [512, 576) uses v_mfma_f32_16x16x32_bf16 with K widened exactly to bf16
//       (every e4m3fn value is a bf16 value) and q in bf16.
//   softmax: online, exp2 domain.  The running max moves only when a score passes
//       it by more than one (log2 units), so p <= 2 and most tiles skip rescaling
//       the accumulator.
//   PV: v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 x e4m3).  P enters as two e4m3
//       terms, hi = e4m3(128 p) and lo = e4m3(16 (128 p - hi)), the lo product
//       scaled by 2^-4 through the MX block scale: about 8 significant bits per
//       probability.  128 p <= 256 never overflows e4m3, and the factor keeps small
//       probabilities out of the subnormal range; it is divided out at the end.
//       The running sum uses the unrounded fp32 p.  The A operand (32 keys of one V
//       column per lane) comes from four ds_read_b64_tr_b8 transposed LDS reads: in
//       each 16-lane group, lanes 2k and 2k+1 address the two 8-byte halves of a
//       16-column slice of key row k, and lane c receives column c of the 8 rows.
//       The 32 keys of lane group j are, in order, the wave's own 16 keys
//       64 hf + 16 s + 4 j + i and then its partner's (s, i < 4): exactly the
//       scores the lane and its partner lane hold, so P needs no reshuffling.

#include <limits.h>
#include <math.h>

#include "va_internal.h"

namespace va {

namespace {

constexpr int kMB = 128;              // keys per tile
constexpr int kLat = 512;             // latent bytes per key (= V)
constexpr int kRope = 64;             // rope bytes per key
constexpr int kNW = 8;                // waves per workgroup
constexpr int kKPW = kMB / kNW;       // keys each wave copies per tile
constexpr int kLatTile = kMB * kLat;
constexpr int kRopeTile = kMB * kRope;
constexpr int kCT = 256 / 16;         // O^T column tiles per wave
constexpr float kPScale = 128.f;      // P scale for e4m3 (p <= 2^kLazy, so 128 p <= 256 < 448)
constexpr float kLazy = 1.f;          // log2 headroom before the running max is moved
constexpr int kE8M0One = 127;         // MX block scale exponents (bias 127)
constexpr int kE8M0Sixteenth = 123;
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Chunk permutation of latent row t (16-byte chunks, XOR inside aligned groups of 16).
__device__ __forceinline__ int lat_swz(int t) { return (t & 15) ^ (((t >> 4) & 1) << 3); }

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

// Copies to LDS at `lds` + lane * 16 straight from global memory.  Inline assembly,
// so the compiler (which does not see these copies) adds no waits of its own before
// LDS reads; the waits are explicit.  M0 holds the wave's LDS base and needs one
// wait state before the copy reads it.  (Non-temporal copies, `nt`, left this compute-
// bound pass's time unchanged and raised its fetched bytes by 19 MB per call.)
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier ordering LDS only: outstanding copies into the ring stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS of the one workgroup a compute unit holds: the two-tile latent ring, the rope
// buffer, and the pair exchanges (probabilities: [wave][hi, lo][lane][16 bytes];
// row maxima and sums: [wave][row]).
__shared__ __attribute__((aligned(128))) uint8_t s_lat[2][kLatTile];
__shared__ __attribute__((aligned(128))) uint8_t s_rope[kRopeTile];
__shared__ __attribute__((aligned(16))) i32x4 s_xp[kNW][2][64];
__shared__ float s_xm[kNW][16];
__shared__ uint32_t s_qex[4][16];  // per row group: the bf16 exponent field E of each q row

}  // namespace

__global__ __launch_bounds__(512) void splitkv_mla_fp8_kernel(FwdParams P) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;
  const int hf = wave >> 2;
  const int partner = wave ^ 4;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.x;
  PieceWalk pw;
  if (!pw.init(P, blockIdx.y)) return;  // uniform over the workgroup, before any barrier

  const int row = rg * 16 + n;
  const bool tree = P.draft_slots != nullptr;
  const uint8_t* kg = P.k + (int64_t)g * P.k_shead;
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;

  // per-lane LDS offsets, fixed for the kernel:
  //   qoff[e][x]: 16-byte half e of the lane's 32-byte K operand slice (row 64 hf + n,
  //            chunks 8 kb + 2 j + e) for token tile tt and k-block kb with
  //            x = (kb ^ tt) % 2; the rest (8192 tt + 256 (kb / 2)) is an immediate;
  //   voff[r]: transposed V read of key slots 8r .. 8r+7 (own keys first), this
  //            wave's columns, the lane's 8-byte half; column tile ct reads at
  //            voff[r] ^ 16 ct (bits 4..7 of voff hold the row's permutation);
  //   roff[h]: rope k-step h of token tile 0 (lane group j: 8 bytes at 32 h + 8 j);
  //   cx:      the lane's source chunk for copy pair 0 (pair i: cx ^ 2 i).
  int qoff[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      qoff[e][x] = kLat * (64 * hf + n) + 16 * ((2 * j + e) ^ (n & 7)) + 128 * ((n >> 3) ^ x);
  int voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k8 = n >> 1;
    const int t = 64 * (hf ^ (r >> 1)) + 16 * (2 * (r & 1) + (k8 >> 2)) + 4 * j + (k8 & 3);
    voff[r] = kLat * t + 256 * hf + 8 * (n & 1) + 16 * lat_swz(t);
  }
  const int cx = (lane & 31) ^ (lane >> 5) ^ ((wave & 1) << 3);
  int roff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    roff[h] = (64 * hf + n) * kRope + 16 * ((2 * h + (j >> 1)) ^ ((n >> 2) & 3)) + 8 * (j & 1);

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
  // (row bounds and tree bits are loaded before any copy is issued, so the
  // compiler's waits for them never count copies in flight)
  // keys of row i: p - W <= t <= p with p = L + i (prefix and causal draft keys)
  const int row_lo = (P.window >= 0 && rv) ? L + row_i - P.window : INT_MIN;
  const int row_hi = rv ? (tree ? t_last : min(t_last, L + row_i)) : -1;
  const uint32_t tbits = (tree && rv) ? tree_bits(P, b, row_i) : 0u;
  // keys every row of the pair sees: key halves inside [wave_lo, wave_hi] need no
  // masking (tree draft keys and capped logits always take the general path)
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

  // key of lane l < 16 among this wave's 16 copies of tile k (clamped to the piece)
  auto copy_key = [&](int k) { return min(t_begin + k * kMB + wave * kKPW + (lane & 15), t_last); };
  // page id of that key, branch-free (a tree-verify draft key reads entry 0 and takes
  // its draft slot in make_slot), so the compiler's waits count this load exactly
  auto load_pid = [&](int k) -> int {
    const int t = copy_key(k);
    const bool draft_key = tree && t >= L;
    const int v = *(const __attribute__((address_space(1))) int32_t*)(bt_row + (draft_key ? 0 : t >> lg));
    return draft_key ? 0 : v;
  };
  // The draft slot of a tree-verify key is one more load: the empty asm takes its
  // wait inside the (uniform) tree branch, before the copies; the plain path waits
  // only for the page id.
  auto make_slot = [&](int pid, int k) -> int {
    const int t = copy_key(k);
    int slot = (pid << lg) | (t & pmask);
    if (tree) {
      int s = *(const __attribute__((address_space(1))) int32_t*)(
          P.draft_slots + b * P.draft + min(max(t - L, 0), P.draft - 1));
      asm volatile("" : "+v"(s));
      slot = t >= L ? s : slot;
    }
    return slot;
  };
  // latent bytes of keys 2i, 2i+1 of this wave's 16 keys of tile k -> ring buffer
  // k % 2, one instruction: lanes 0..31 copy the first key's row, lanes 32..63 the
  // second's, lane l into chunk position l % 32 (which holds chunk (l % 32) ^ f(t))
  auto copy_pair = [&](int k, int slot_l, int i) {
    const int s0 = __builtin_amdgcn_readlane(slot_l, 2 * i);
    const int s1 = __builtin_amdgcn_readlane(slot_l, 2 * i + 1);
    int slot = lane < 32 ? s0 : s1;
    // ordered after the previous copy, so the address math is not hoisted (and held
    // in registers) ahead of it
    asm volatile("" : "+v"(slot));
    dma16(kg + (int64_t)slot * P.k_sslot + 16 * (cx ^ (2 * i)),
          lds_addr(s_lat[k & 1] + (wave * kKPW + 2 * i) * kLat));
  };
  // rope bytes of this wave's keys -> rope buffer, one instruction: lane l copies
  // chunk l % 4 position of key l / 4 (chunks permuted per row against bank conflicts)
  auto copy_rope = [&](int slot_l) {
    const int u = lane >> 2;
    const int s = __shfl(slot_l, u, 64);
    const int c = (lane & 3) ^ ((u >> 2) & 3);
    dma16(kg + (int64_t)s * P.k_sslot + kLat + 16 * c, lds_addr(s_rope + wave * kKPW * kRope));
  };

  int pid = 0, slot_nx = 0;
  // This pair's 16 q rows in registers, scaled per row by 2^(134 - E) with E the bf16
  // exponent field of the row's largest magnitude (latent and rope, at least 8), which
  // puts that magnitude in [128, 256) whatever the range of q; the scores are scaled
  // back by 2^(E - 134) with sm_scale.  For d < 512 the scaled q x is held as two e4m3
  // terms, hi = e4m3(x) and lo = e4m3(x - hi): hi is off by at most 8 near the row's
  // largest elements, where lo is a normal e4m3 number, so the pair carries ~2^-9 of
  // the row's largest magnitude, the precision of the bf16 q itself.  The 64-wide
  // rope tail d >= 512 stays bf16 (scaled exactly).  Lane group j holds elements
  // 128kb + 32j + [0, 32) (and 512 + 32h + 8j + [0, 8) of the tail), the k-slots of
  // the K operand read below.
  // Each wave of the pair loads and converts 8 of the 16 rows (lane l: row
  // 8 hf + l % 8, elements 64 (l / 8) + [0, 64) and 8 rope elements), so the row's
  // exponent is found inside the wave, and hands the terms to both waves through ring
  // buffer 1, which tile 1 fills only later.  The page ids of tiles 0 and 1 are loaded
  // first, so the copies of tile 0 wait only for them and are in flight together with q.
  i32x8 qh[kLat / 128], ql[kLat / 128];
  u32x4 qr[2];
  float c_row;  // sm_scale * k_scale * log2(e) * 2^(E - 134) of the lane's row
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // rows past the sequence's count read q row 0 (always present) and are zeroed
    auto q_row = [&](int r, bool ok) -> const uint8_t* {
      return ok ? P.q + (int64_t)(seq_row0(P, b) + r / P.group) * P.q_srow +
                      (int64_t)(g * P.group + r % P.group) * P.q_shead
                : P.q;
    };
    const int crow = rg * 16 + 8 * hf + (lane & 7);  // the row this lane converts
    const int cc = lane >> 3;                         // its 64-element chunk
    const bool cv = crow < P.rows && crow / P.group < seq_rows(P, b);
    const uint8_t* qc = q_row(crow, cv);
    const uint8_t* qp = q_row(row, rv);
    const int pid0 = load_pid(0);
    pid = load_pid(1);
    u32x4 raw[9];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const u32x4*>(qc + 2 * (64 * cc + 8 * i));
    raw[8] = *reinterpret_cast<const u32x4*>(qc + 2 * (kLat + 8 * cc));
#pragma unroll
    for (int h = 0; h < 2; ++h) qr[h] = *reinterpret_cast<const u32x4*>(qp + 2 * (kLat + 32 * h + 8 * j));
    slot_nx = make_slot(pid0, 0);
#pragma unroll
    for (int i = 0; i < kKPW / 2; ++i) copy_pair(0, slot_nx, i);
    copy_rope(slot_nx);
    // the conversion stays after the copies (its wait for q then counts them too)
#pragma unroll
    for (int i = 0; i < 9; ++i) asm volatile("" : "+v"(raw[i]));
#pragma unroll
    for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(qr[h]));
#pragma unroll
    for (int i = 0; i < 9; ++i) raw[i] = cv ? raw[i] : zero;
#pragma unroll
    for (int h = 0; h < 2; ++h) qr[h] = rv ? qr[h] : zero;
    // the row's largest magnitude: bf16 bit patterns without the sign compare as the
    // magnitudes do; the 8 lanes l % 8 of a row hold its 512 + 64 elements
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 9; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = max(amax, max(raw[i][e] & 0x7fffu, (raw[i][e] >> 16) & 0x7fffu));
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
    const uint32_t ex = min(max(amax >> 7, 8u), 254u);
    const float mult = __uint_as_float((261u - ex) << 23);  // 2^(134 - E)
    // Terms to ring buffer 1, pair region [hi, lo][kb][lane n + 16 j][32 bytes]: this
    // lane's elements 64 cc + [0, 32) are block kb = cc / 2 of lane group 2 (cc % 2),
    // the next 32 of lane group 2 (cc % 2) + 1.
    uint8_t* xo = s_lat[1] + 16384 * rg + 2048 * (cc >> 1) + 32 * ((crow & 15) + 32 * (cc & 1));
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      i32x4 th[2], tl[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 r = raw[4 * hv + i];
        float x[8];  // scaled q elements: exact, magnitudes below 256
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(r[e] << 16) * mult;
          x[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u) * mult;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h], x[4 * h + 1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h + 2], x[4 * h + 3], w, true);
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          const f32x2 c2 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
          int wl = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h] - a[0], x[4 * h + 1] - a[1], 0, false);
          wl = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h + 2] - c2[0], x[4 * h + 3] - c2[1], wl, true);
          th[i >> 1][2 * (i & 1) + h] = w;
          tl[i >> 1][2 * (i & 1) + h] = wl;
        }
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        *reinterpret_cast<i32x4*>(xo + 512 * hv + 16 * q2) = th[q2];
        *reinterpret_cast<i32x4*>(xo + 8192 + 512 * hv + 16 * q2) = tl[q2];
      }
    }
    if (cc == 0) s_qex[rg][crow & 15] = ex;
    lds_barrier();
    const uint8_t* xi = s_lat[1] + 16384 * rg + 32 * lane;
#pragma unroll
    for (int kb = 0; kb < kLat / 128; ++kb) {
      const u32x4 h0 = *reinterpret_cast<const u32x4*>(xi + 2048 * kb);
      const u32x4 h1 = *reinterpret_cast<const u32x4*>(xi + 2048 * kb + 16);
      const u32x4 l0 = *reinterpret_cast<const u32x4*>(xi + 8192 + 2048 * kb);
      const u32x4 l1 = *reinterpret_cast<const u32x4*>(xi + 8192 + 2048 * kb + 16);
      qh[kb] = __builtin_bit_cast(i32x8, u32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
      ql[kb] = __builtin_bit_cast(i32x8, u32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]});
    }
    const uint32_t rex = s_qex[rg][n];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float rmult = __uint_as_float((261u - rex) << 23);
    c_row = P.c_log2 * __uint_as_float((rex - 7u) << 23);
    // the rope tail in bf16, scaled by the same power of two (exact)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = qr[h][e];
        const uint32_t lo16 = __float_as_uint(__uint_as_float(w << 16) * rmult) >> 16;
        const uint32_t hi16 = __float_as_uint(__uint_as_float(w & 0xffff0000u) * rmult) & 0xffff0000u;
        qr[h][e] = hi16 | lo16;
      }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[kCT];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < ntile; ++k) {
    // this wave's copies of tile k (and page ids of tile k + 1) have landed; the
    // barrier shows every wave's and frees the ring buffer tile k - 1 was read from
    wait_copies();
    lds_barrier();
    // compiler-visible loads go before the copies: a wait the compiler places for
    // them then never counts the copies still in flight
    const bool next = k + 1 < ntile;
    if (next) slot_nx = make_slot(pid, k + 1);
    pid = load_pid(k + 2);  // clamped to the piece's last key past its end

    const int t0 = t_begin + k * kMB;
    const int th = t0 + 64 * hf;  // first key this wave scores
    const uint8_t* lat = s_lat[k & 1];

    // a4: S^T for the wave's 4 token tiles of 16 keys
    f32x4 sacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // d < 512: fp8 x fp8 (K bytes as they are, q as hi + lo terms), in 8 operand groups
    // g = (kb, token-tile pair): the two 16-key operands of group g + 1 are read from
    // LDS before the four products of group g issue, so their latency runs under the
    // matrix instructions.  Token tiles go in pairs so the two products into one
    // accumulator are not back to back.
    auto k_operands = [&](int g, i32x8* ka) {
      const int kb = g >> 1, tt = 2 * (g & 1);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int x = (kb ^ (tt + e)) & 1;
        const int imm = 8192 * (tt + e) + 256 * (kb >> 1);
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(lat + qoff[0][x] + imm);
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(lat + qoff[1][x] + imm);
        ka[e] = __builtin_bit_cast(i32x8, u32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]});
      }
    };
    // rope operands (bf16 k-steps, lane group j holds 512 + 32h + 8j + [0, 8)), read
    // with the last latent group
    u32x2 kr[2][4];
    i32x8 kc[2], kn[2];
    k_operands(0, kc);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int kb = g >> 1, tt = 2 * (g & 1);
      if (g < 7) {
        k_operands(g + 1, kn);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4)
            kr[h][t4] = *reinterpret_cast<const u32x2*>(s_rope + roff[h] + 16 * kRope * t4);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        sacc[tt + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[e], qh[kb], sacc[tt + e], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        sacc[tt + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[e], ql[kb], sacc[tt + e], 0, 0, 0, 0, 0, 0);
      // one copy of the next tile per operand group (8 per tile)
      if (next) copy_pair(k + 1, slot_nx, g);
      __builtin_amdgcn_sched_barrier(0);
      kc[0] = kn[0];
      kc[1] = kn[1];
    }
    // rope tail d in [512, 576): bf16 products with K widened exactly
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const u32x2 w0 = fp8x4_to_bf16x4(kr[h][tt][0]), w1 = fp8x4_to_bf16x4(kr[h][tt][1]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]}), as_bf16x8(qr[h]), sacc[tt], 0, 0, 0);
      }
    }

    // the lane's 16 scores of row n: slot e is key th + 16 (e / 4) + 4 j + e % 4
    float sc[16];
    float bmax = -INFINITY;
    if (th >= wave_lo && th + 63 <= wave_hi) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[e] = sacc[e >> 2][e & 3] * c_row;
        bmax = fmaxf(bmax, sc[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = th + 16 * (e >> 2) + 4 * j + (e & 3);
        const bool ok = key_ok(t, row_lo, row_hi, L, tbits, tree);
        sc[e] = ok ? sacc[e >> 2][e & 3] * c_row : -INFINITY;
      }
      if (P.logit_cap > 0.f) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = sc[e] == -INFINITY ? sc[e] : cap_log2(sc[e], P.logit_cap);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, sc[e]);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    if (j == 0) s_xm[wave][n] = bmax;
    // every wave's maxima are written and every rope read of tile k is done
    lds_barrier();
    if (next) copy_rope(slot_nx);
    bmax = fmaxf(bmax, s_xm[partner][n]);

    // the reference max moves only when a score passes it by more than kLazy, so
    // most tiles leave the accumulator alone; p = 2^(s - m) stays <= 2^kLazy.  Both
    // waves of the pair take the same decision from the same maxima.
    const bool grow = bmax > m_run + kLazy;
    const float m_new = grow ? bmax : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += sc[e];
    }
    // P in two e4m3 terms: hi = e4m3(128 p), lo = e4m3(16 (128 p - hi)); the lo
    // product enters the same accumulator through the MFMA's B scale 2^-4
    i32x4 ph, pl;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float x0 = sc[4 * d] * kPScale, x1 = sc[4 * d + 1] * kPScale;
      const float x2 = sc[4 * d + 2] * kPScale, x3 = sc[4 * d + 3] * kPScale;
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
      ph[d] = w;
      const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      int wl = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - h01[0]) * 16.f, (x1 - h01[1]) * 16.f, 0, false);
      wl = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - h23[0]) * 16.f, (x3 - h23[1]) * 16.f, wl, true);
      pl[d] = wl;
    }
    s_xp[wave][0][lane] = ph;
    s_xp[wave][1][lane] = pl;
    // the pair's probabilities are written
    lds_barrier();
    const i32x4 qph = s_xp[partner][0][lane];
    const i32x4 qpl = s_xp[partner][1][lane];
    const i32x8 pb = i32x8{ph[0], ph[1], ph[2], ph[3], qph[0], qph[1], qph[2], qph[3]};
    const i32x8 pb_lo = i32x8{pl[0], pl[1], pl[2], pl[3], qpl[0], qpl[1], qpl[2], qpl[3]};

    // rescale only when some row with a nonzero accumulator moved its max
    if (__any(grow && m_run != -INFINITY)) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) oacc[ct] *= alpha;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // a5: O^T += V^T P^T over all 128 keys, this wave's 256 columns, two column tiles
    // per step: the V^T operands of step s + 1 are read from LDS before the four
    // products of step s issue
    __attribute__((address_space(3))) char* lbase = (__attribute__((address_space(3))) char*)lat;
    auto v_operands = [&](int ct, i32x8* a) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              reinterpret_cast<lds_i32x2*>(lbase + (voff[r] ^ (16 * (ct + e)))));
          a[e][2 * r] = x[0];
          a[e][2 * r + 1] = x[1];
        }
      }
    };
    i32x8 vc[2], vn[2];
    v_operands(0, vc);
#pragma unroll
    for (int ct = 0; ct < kCT; ct += 2) {
      if (ct + 2 < kCT) v_operands(ct + 2, vn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        oacc[ct + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vc[e], pb, oacc[ct + e], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        oacc[ct + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vc[e], pb_lo, oacc[ct + e], 0, 0, 0,
                                                                        kE8M0One, 0, kE8M0Sixteenth);
      __builtin_amdgcn_sched_barrier(0);
      vc[0] = vn[0];
      vc[1] = vn[1];
    }
  }

  // each lane summed only its own keys: total the 4 lanes of the row, then the pair
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (j == 0) s_xm[wave][n] = l_run;
  lds_barrier();
  l_run += s_xm[partner][n];
  if (rv) {
    const int64_t split_id = ((int64_t)b * P.hkv + g) * P.slots + pc.slot;
    const float inv = l_run > 0.f ? P.v_scale / (l_run * kPScale) : 0.f;
    float* po = P.part_o + (split_id * P.rows + row) * kLat + 256 * hf + 4 * j;
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      f32x4 o = oacc[ct];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= inv;
      *reinterpret_cast<f32x4*>(po + 16 * ct) = o;
    }
    if (hf == 0 && j == 0)
      P.part_lse[split_id * P.rows + row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
  // every wave is done with the ring, the rope buffer and the exchanges before the
  // next piece refills them
  lds_barrier();
  } while (pw.next(P));
}

int launch_splitkv_mla_fp8(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t st) {
  if (p.rows > 64) return VA_EUNSUPPORTED;
  return launch_kernel(reinterpret_cast<const void*>(&splitkv_mla_fp8_kernel), grid, dim3(kNW * 64),
                       fp, st);
}

}  // namespace va
