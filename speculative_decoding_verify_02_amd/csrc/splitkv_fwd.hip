// Split-KV (flash-decode) pass over the prefix for EAGLE target-verify at topk = 1.
//
// PR #27382 ("[AMD][Perf] Split-KV flash-decode attention for EAGLE target-verify",
// sections "Motivation" and "Modifications") splits the long shared prefix across
// parallel programs, each writing a partial output and log-sum-exp that a second
// stage merges.  This is the gfx950 design of that first stage:
//
//   workgroup = (head group, key range y), 4 waves of 64 lanes; the range is cut
//   at sequence ends into pieces (see PieceWalk), each attended in turn.
//   All G*D query rows of a KV head form the dense M dimension (16/32/64 rows).
//   The 4 waves cover HPC KV heads x NRG row groups (16*RT rows each) x NTL token
//   lanes; token lanes of one (head, row group) interleave the piece's blocks and
//   merge through LDS at the end.  The grid runs head groups fastest, so the heads
//   of one token range are read at about the same time (DRAM locality).
//
// Per block of 16*TT tokens a wave
//   1. maps its tokens to slots through the block table (one page-id load per lane,
//      fetched a block ahead and spread with ds_bpermute),
//   2. loads K rows coalesced (whole rows per instruction) and stages them in a
//      private padded LDS tile, from which it reads the MFMA A operand (lane l:
//      token l%16, 16 bytes at 64*u + 16*(l/16) of the row),
//   3. loads V rows coalesced straight into registers: the lane keeps 16-byte groups
//      (256 bytes apart) of its 4*TT score-slot tokens,
//   4. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp8 K is widened to
//      bf16 exactly in registers), so each lane ends up with scores of ONE row,
//   5. runs the online softmax in the exp2 domain (row max across the 4 lanes of a
//      row by two xor-shuffles, running sum kept per lane),
//   6. computes O^T += V^T P^T: the lane's own probabilities are the B operand (no
//      data movement) and V^T's A operand is a transpose inside the lane's
//      registers (the column permutation is undone when the partial is written).
// For d = 128 the next block's K/V loads are in flight while a block computes.
// The last wave of each (head, row group) writes the piece's partial O (normalised,
// times v_scale) and LSE (natural log) to the workspace.
//
// Masking: row i (position p = L + i) keeps keys p - W <= t <= p, so later draft
// keys are causal-masked and, with a left window W, old prefix keys too.  Masked
// scores are set to -inf by selection; token loads past the piece are clamped to
// its last real token so no load leaves the sequence.

#include <limits.h>
#include <math.h>

#include "va_internal.h"

namespace va {


namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// 4 fp8 e4m3fn bytes -> 4 bf16 (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t x) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Block geometry for one KV head: K rows of qk_dim elements, V rows of v_dim.
template <int DK, int DV, bool FP8, int TT>
struct Geo {
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int TB = 16 * TT;            // tokens per block
  static constexpr int KRB = DK * EB;           // K row bytes
  static constexpr int KCH = KRB / 16;          // 16-byte chunks per K row
  static constexpr int NKLD = TB * KCH / 64;    // coalesced K loads per lane per block
  static constexpr int RS = KRB + 16;           // LDS row stride; +16 keeps reads conflict-free
  static constexpr int TILE = TB * RS;          // LDS bytes of one wave's K tile
  static constexpr int KU = KRB / 64;           // 16-byte operand chunks per lane per token
  static constexpr int KSTEPS = DK / 32;        // MFMA k-steps
  static constexpr int VRB = DV * EB;           // V row bytes read
  static constexpr int VG = VRB >= 256 ? VRB / 256 : 1;   // V groups per lane per token
  static constexpr int VGB = VRB >= 256 ? 16 : VRB / 16;  // bytes per group
  static constexpr int VW = VG * VGB / 4;       // V dwords per lane per token
  static constexpr int EPG = VGB / EB;          // V elements per group
  static constexpr int CG = 256 / EB;           // elements spanned by one 256-byte group stride
  static constexpr int CPL = DV / 16;           // O^T column tiles = V columns per lane
  static_assert((TB * KCH) % 64 == 0, "whole K loads per block");
  static_assert(CPL == VG * EPG, "V groups cover the lane's columns");
  static_assert(KRB % 64 == 0, "K operand chunks");
};

template <class G>
struct KVRegs {
  u32x4 k[G::NKLD];               // coalesced K chunks, staged to LDS
  uint32_t v[4 * G::TB / 16][G::VW];  // V groups of the lane's score-slot tokens
};

// Token of S^T slot i (0 .. 4*TT-1) of lane group j: the 16x16 accumulator of token
// tile tt holds tokens 16*tt + 4*j + r (r = 0..3) in a lane.  P^T and V^T use the
// same slot order, which is all the MFMA reduction needs.
__device__ __forceinline__ int slot_token(int j, int i) { return 16 * (i >> 2) + 4 * j + (i & 3); }

// The K and V rows are read once per call: non-temporal loads, so the stream does not
// displace what is reused (page ids, q, the partials the combine reads back) from the
// L2s and the Infinity Cache.  On the long-context batch this took the pass from 397 to
// 357 us; making the partial stores non-temporal as well cost 50 us.
template <class G>
__device__ __forceinline__ void load_block(KVRegs<G>& R, int lslot, const uint8_t* kg,
                                           const uint8_t* vg, uint32_t k_sslot, uint32_t v_sslot,
                                           int lane, int n, int j) {
#pragma unroll
  for (int u = 0; u < G::NKLD; ++u) {
    const int q = 64 * u + lane;
    const int sl = __shfl(lslot, q / G::KCH, 64);
    R.k[u] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(kg + (uint64_t)(uint32_t)sl * k_sslot + 16 * (q % G::KCH)));
  }
#pragma unroll
  for (int i = 0; i < 4 * G::TB / 16; ++i) {
    const int sl = __shfl(lslot, slot_token(j, i), 64);
    const uint8_t* vp = vg + (uint64_t)(uint32_t)sl * v_sslot + G::VGB * n;
#pragma unroll
    for (int c = 0; c < G::VG; ++c) {
      if constexpr (G::VGB == 16) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 256 * c));
        R.v[i][4 * c + 0] = x[0];
        R.v[i][4 * c + 1] = x[1];
        R.v[i][4 * c + 2] = x[2];
        R.v[i][4 * c + 3] = x[3];
      } else {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp));
        R.v[i][0] = x[0];
        R.v[i][1] = x[1];
      }
    }
  }
}

// K chunks -> the wave's LDS tile (row-major, stride RS).
template <class G>
__device__ __forceinline__ void stage_k(const KVRegs<G>& R, uint8_t* tile, int lane) {
#pragma unroll
  for (int u = 0; u < G::NKLD; ++u) {
    const int q = 64 * u + lane;
    *reinterpret_cast<u32x4*>(tile + (q / G::KCH) * G::RS + 16 * (q % G::KCH)) = R.k[u];
  }
}

// Per-wave running state of the online softmax for RT row tiles.
template <int DV, int RT>
struct RowState {
  float m[RT], l[RT];
  f32x4 o[RT][DV / 16];
};

// Per-piece key masks of a wave's RT row tiles (lane's row n of each).
template <int RT>
struct RowMask {
  int lo[RT], hi[RT];   // key range p - W .. p of the row (p = L + i)
  uint32_t bits[RT];    // tree verify: draft keys the row sees
  int L;                // first draft key
  bool tree;
  float c_log2;         // sm_scale * k_scale * log2(e)
  float cap;            // logit cap (0: off)
};

template <class G, bool FP8, int RT, int DV, bool EXT>
__device__ __forceinline__ void compute_block(const uint8_t* tile, const KVRegs<G>& R,
                                              const bf16x8 (&qB)[RT][G::KSTEPS],
                                              const RowMask<RT>& mk, RowState<DV, RT>& st, int t0,
                                              int n, int j) {
  constexpr int TT = G::TB / 16;
  constexpr int NS = 4 * TT;  // scores per lane per row tile
  constexpr int CPL = G::CPL;

  // a4: S^T = K Q^T, K operand chunks read from the LDS tile
  f32x4 sacc[TT][RT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sacc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ku = 0; ku < G::KU; ++ku) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const u32x4 c =
          *reinterpret_cast<const u32x4*>(tile + (16 * tt + n) * G::RS + 64 * ku + 16 * j);
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2 w0 = fp8x4_to_bf16x4(c[2 * h]);
          const u32x2 w1 = fp8x4_to_bf16x4(c[2 * h + 1]);
          const bf16x8 a = as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            sacc[tt][rt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[rt][2 * ku + h], sacc[tt][rt], 0, 0, 0);
        }
      } else {
        const bf16x8 a = as_bf16x8(c);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[rt][ku], sacc[tt][rt], 0, 0, 0);
      }
    }
  }

  // online softmax in the exp2 domain; the lane holds NS scores of one row per tile
  uint32_t pbits[RT][NS / 2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float sc[NS];
    float bmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      const int t = t0 + 16 * (e >> 2) + 4 * j + (e & 3);
      bool ok;
      if constexpr (EXT) ok = key_ok(t, mk.lo[rt], mk.hi[rt], mk.L, mk.bits[rt], mk.tree);
      else ok = (t >= mk.lo[rt]) && (t <= mk.hi[rt]);
      sc[e] = ok ? sacc[e >> 2][rt][e & 3] * mk.c_log2 : -INFINITY;
    }
    if constexpr (EXT) {
      if (mk.cap > 0.f) {
#pragma unroll
        for (int e = 0; e < NS; ++e) sc[e] = sc[e] == -INFINITY ? sc[e] : cap_log2(sc[e], mk.cap);
      }
    }
#pragma unroll
    for (int e = 0; e < NS; ++e) bmax = fmaxf(bmax, sc[e]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(st.m[rt], bmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m[rt] - m_use);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += sc[e];
    }
    st.l[rt] = st.l[rt] * alpha + psum;
    st.m[rt] = m_new;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) st.o[rt][ct] *= alpha;
#pragma unroll
    for (int e = 0; e < NS; e += 2) {
      const __bf16 lo = (__bf16)sc[e], hi = (__bf16)sc[e + 1];
      pbits[rt][e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  }

  // a5: O^T += V^T P^T.  Column tile ct = (group c, element e) holds, in row m,
  // column c*CG + EPG*m + e.
#pragma unroll
  for (int ct = 0; ct < CPL; ++ct) {
    const int c = ct / G::EPG, e = ct % G::EPG;
    uint32_t av[NS / 2];
    if constexpr (FP8) {
      const int w = c * (G::VGB / 4) + e / 4, sh = 8 * (e & 3);
#pragma unroll
      for (int h = 0; h < NS / 4; ++h) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) x |= ((R.v[4 * h + k][w] >> sh) & 0xffu) << (8 * k);
        const u32x2 cv = fp8x4_to_bf16x4(x);
        av[2 * h] = cv[0];
        av[2 * h + 1] = cv[1];
      }
    } else {
      const int w = c * (G::VGB / 4) + e / 2;
#pragma unroll
      for (int q2 = 0; q2 < NS / 2; ++q2) {
        const uint32_t a0 = R.v[2 * q2][w], a1 = R.v[2 * q2 + 1][w];
        av[q2] = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (TT == 2) {
        st.o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(u32x4{av[0], av[1], av[2], av[3]}),
            as_bf16x8(u32x4{pbits[rt][0], pbits[rt][1], pbits[rt][2], pbits[rt][3]}),
            st.o[rt][ct], 0, 0, 0);
      } else {
        st.o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(s16x4, u32x2{av[0], av[1]}),
            __builtin_bit_cast(s16x4, u32x2{pbits[rt][0], pbits[rt][1]}), st.o[rt][ct], 0, 0, 0);
      }
    }
  }
}

}  // namespace

// EXT: tree verify and logit cap compiled in (they cost registers the plain path
// needs, so the plain instances leave them out).
template <int DK, int DV, bool FP8, int RT, int NRG, int NTL, int TT, bool PIPE, int WPE, bool EXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
void splitkv_fwd_kernel(FwdParams P) {
  using G = Geo<DK, DV, FP8, TT>;
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int CPL = G::CPL;
  constexpr int HPC = kWaves / (NRG * NTL);
  constexpr int TB = G::TB;
  static_assert(HPC * NRG * NTL == kWaves, "wave layout");
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[kWaves][G::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int hc = wave / (NRG * NTL);
  const int rg = (wave / NTL) % NRG;
  const int tl = wave % NTL;
  const int g = blockIdx.x * HPC + hc;     // KV head of this wave
  const bool head_ok = g < P.hkv;          // the last head group may be partial
  PieceWalk pw;
  if (!pw.init(P, blockIdx.y)) return;  // uniform over the workgroup, before any barrier
  const uint8_t* kg = P.k + (int64_t)g * P.k_shead;
  const uint8_t* vg = P.v + (int64_t)g * P.v_shead;
  // slot s's row is s * sslot bytes in (the host checks that a slot stride fits in 32 bits)
  const uint32_t k_sslot = (uint32_t)P.k_sslot, v_sslot = (uint32_t)P.v_sslot;
  uint8_t* tile = s_tile[wave];
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;

  do {
  const Piece pc = pw.piece(P);
  const int b = pc.b;
  const int L = pc.L;
  const int t_begin = pc.t0, t_end = pc.t1;
  const int nblk = head_ok ? (t_end - t_begin + TB - 1) / TB : 0;
  const int t_last = t_end - 1;
  if (pc.count > 0 && blockIdx.x == 0 && threadIdx.x == 0) P.counts[b] = pc.count;

  // Q^T as the B operand: lane holds row n of each row tile, 8 consecutive k-slots.
  // Keys of row i: p - W <= t <= p with p = L + i (prefix and causal draft keys).
  bf16x8 qB[RT][KSTEPS];
  RowMask<RT> mk;
  mk.L = L;
  mk.tree = P.draft_slots != nullptr;
  mk.c_log2 = P.c_log2;
  mk.cap = P.logit_cap;
  const int nrow_b = seq_rows(P, b), row0_b = seq_row0(P, b);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (rg * RT + rt) * 16 + n;
    const int i0 = row / P.group;
    const bool rv = head_ok && row < P.rows && i0 < nrow_b;
    const int i = rv ? i0 : 0;
    const int hh = rv ? row % P.group : 0;
    mk.lo[rt] = P.window >= 0 ? L + i - P.window : INT_MIN;
    mk.hi[rt] = rv ? (mk.tree ? t_last : min(t_last, L + i)) : -1;
    mk.bits[rt] = (EXT && mk.tree && rv) ? tree_bits(P, b, i) : 0u;
    const uint8_t* qp =
        P.q + (int64_t)(row0_b + i) * P.q_srow + (int64_t)(g * P.group + hh) * P.q_shead;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      // element offset of this lane's 8 k-slots; matches the K operand chunk layout
      const int d0 = FP8 ? (64 * (ks / 2) + 16 * j + 8 * (ks % 2)) : (32 * ks + 8 * j);
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (rv) raw = *reinterpret_cast<const u32x4*>(qp + 2 * d0);
      qB[rt][ks] = as_bf16x8(raw);
    }
  }

  RowState<DV, RT> st;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st.m[rt] = -INFINITY;
    st.l[rt] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) st.o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;
  auto t0_of = [&](int bk) { return t_begin + bk * TB; };
  // slot of key t0 + (lane % TB), clamped to the piece: one lookup per lane covers a
  // whole block; other lanes read it with ds_bpermute
  auto lslot = [&](int t0) {
    const int t = min(t0 + (lane & (TB - 1)), t_last);
    if constexpr (EXT) return key_slot(P, bt_row, b, L, t, lg, pmask);
    else return (bt_row[t >> lg] << lg) | (t & pmask);
  };

  // a3: this wave's blocks are tl, tl+NTL, ...
  int blk = tl;
  if (blk < nblk) {
    if constexpr (PIPE) {
      // Block blk + NTL's K/V loads are in flight while block blk computes (register
      // sets A/B).  A page-id lookup is issued before the data loads of the block
      // before it and used a half step later, so the compiler's wait for it never
      // counts data loads still in flight.  The steps have no branches: a block past
      // the piece loads its last token (a valid address) and is never computed
      // masked, so the compiler keeps exact counts of the loads in flight.  The loop
      // takes blocks in pairs; a last odd block is computed after it.
      auto lraw = [&](int t0) -> int {
        const int t = min(t0 + (lane & (TB - 1)), t_last);
        const int32_t* src = (EXT && mk.tree && t >= L) ? P.draft_slots + b * P.draft + (t - L)
                                                        : bt_row + (t >> lg);
        return *(const __attribute__((address_space(1))) int32_t*)src;
      };
      auto rslot = [&](int raw, int t0) -> int {
        const int t = min(t0 + (lane & (TB - 1)), t_last);
        return (EXT && mk.tree && t >= L) ? raw : (raw << lg) | (t & pmask);
      };
      KVRegs<G> A, Bk;
      const int raw0 = lraw(t0_of(blk));
      int raw1 = lraw(t0_of(blk + NTL));
      load_block<G>(A, rslot(raw0, t0_of(blk)), kg, vg, k_sslot, v_sslot, lane, n, j);
      int raw2 = lraw(t0_of(blk + 2 * NTL));
      stage_k<G>(A, tile, lane);
      for (; blk + NTL < nblk; blk += 2 * NTL) {
        load_block<G>(Bk, rslot(raw1, t0_of(blk + NTL)), kg, vg, k_sslot, v_sslot, lane, n, j);
        raw1 = lraw(t0_of(blk + 3 * NTL));
        compute_block<G, FP8, RT, DV, EXT>(tile, A, qB, mk, st, t0_of(blk), n, j);
        stage_k<G>(Bk, tile, lane);
        load_block<G>(A, rslot(raw2, t0_of(blk + 2 * NTL)), kg, vg, k_sslot, v_sslot, lane, n, j);
        raw2 = lraw(t0_of(blk + 4 * NTL));
        compute_block<G, FP8, RT, DV, EXT>(tile, Bk, qB, mk, st, t0_of(blk + NTL), n, j);
        stage_k<G>(A, tile, lane);
      }
      // an odd block count leaves one block, already staged in A
      if (blk < nblk) compute_block<G, FP8, RT, DV, EXT>(tile, A, qB, mk, st, t0_of(blk), n, j);
    } else {
      int sl = lslot(t0_of(blk));
      for (; blk < nblk; blk += NTL) {
        KVRegs<G> A;
        load_block<G>(A, sl, kg, vg, k_sslot, v_sslot, lane, n, j);
        if (blk + NTL < nblk) sl = lslot(t0_of(blk + NTL));
        stage_k<G>(A, tile, lane);
        compute_block<G, FP8, RT, DV, EXT>(tile, A, qB, mk, st, t0_of(blk), n, j);
      }
    }
  }

  float (&m_run)[RT] = st.m;
  float (&l_run)[RT] = st.l;
  f32x4 (&oacc)[RT][CPL] = st.o;

  // each lane summed only its own tokens: total the 4 lanes of a row
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16, 64);
    l_run[rt] += __shfl_xor(l_run[rt], 32, 64);
  }

  if constexpr (NTL > 1) {
    // merge the token lanes of each (head, row group) in a fixed order through LDS
    constexpr int NREG = RT * CPL * 4 + RT;
    constexpr int NGRP = HPC * NRG;
    const int grp = hc * NRG + rg;
    __shared__ float sm_m[kWaves][RT][16];
    __shared__ float sm_o[NGRP][NREG][64];
    if (j == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sm_m[wave][rt][n] = m_run[rt];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < NTL; ++k) M = fmaxf(M, sm_m[grp * NTL + k][rt][n]);
      const float f = (m_run[rt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[rt] - M);
      l_run[rt] *= f;
#pragma unroll
      for (int ct = 0; ct < CPL; ++ct) oacc[rt][ct] *= f;
      m_run[rt] = M;
    }
#pragma unroll
    for (int k = 0; k < NTL; ++k) {
      if (tl == k) {
        if (k > 0) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) oacc[rt][ct][r] += sm_o[grp][(rt * CPL + ct) * 4 + r][lane];
            l_run[rt] += sm_o[grp][RT * CPL * 4 + rt][lane];
          }
        }
        if (k < NTL - 1) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) sm_o[grp][(rt * CPL + ct) * 4 + r][lane] = oacc[rt][ct][r];
            sm_o[grp][RT * CPL * 4 + rt][lane] = l_run[rt];
          }
        }
      }
      __syncthreads();
    }
  }

  // write the piece's partial (the last token lane of each (head, row group)).
  // Lane holds row n; for group c and r = 0..3 the columns c*CG + EPG*(4*j + r) + [0, EPG).
  const int64_t split_id = ((int64_t)b * P.hkv + g) * P.slots + pc.slot;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (tl != NTL - 1 || !head_ok) break;
    const int row = (rg * RT + rt) * 16 + n;
    if (row >= P.rows || row / P.group >= nrow_b) continue;
    const float l = l_run[rt];
    const float inv = l > 0.f ? P.v_scale / l : 0.f;
    float* po = P.part_o + (split_id * P.rows + row) * DV;
#pragma unroll
    for (int c = 0; c < G::VG; ++c) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int e4 = 0; e4 < G::EPG; e4 += 4) {
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = oacc[rt][c * G::EPG + e4 + e][r] * inv;
          *reinterpret_cast<f32x4*>(po + c * G::CG + G::EPG * (4 * j + r) + e4) = o;
        }
      }
    }
    if (j == 0)
      P.part_lse[split_id * P.rows + row] = l > 0.f ? (m_run[rt] + log2f(l)) * kLn2 : -INFINITY;
  }
  } while (pw.next(P));
}

namespace {

// Kernel variant per wave layout.  d = 128: 32-token blocks, K/V double-buffered.
// d = 256: 32-token blocks, single buffer (a second one would not fit beside the
// 32x256 accumulator).  d = 576/512: 16-token blocks, single buffer.
template <int DK, int DV, bool FP8, bool EXT>
int launch_dims(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t st) {
  constexpr int TT = DK >= 576 ? 1 : 2;
  constexpr bool PIPE = DK == 128;
  // with one 16-row tile the double-buffered d = 128 kernel fits two waves per SIMD
#define VA_LAUNCH(RT_, NRG_, NTL_)                                                              \
  return launch_kernel(reinterpret_cast<const void*>(                                           \
                           &splitkv_fwd_kernel<DK, DV, FP8, RT_, NRG_, NTL_, TT, PIPE,          \
                                               (DK == 128 && RT_ == 1) ? 2 : 1, EXT>),          \
                       grid, dim3(256), fp, st)
  const int key = p.rt * 100 + p.nrg * 10 + p.ntl;
  if constexpr (DV > 256) {
    // a 512-wide O^T already fills 128 accumulator registers: one row tile per wave
    switch (key) {
      case 111: VA_LAUNCH(1, 1, 1);
      case 112: VA_LAUNCH(1, 1, 2);
      case 114: VA_LAUNCH(1, 1, 4);
      case 121: VA_LAUNCH(1, 2, 1);
      case 122: VA_LAUNCH(1, 2, 2);
      case 141: VA_LAUNCH(1, 4, 1);
      default: return VA_EUNSUPPORTED;
    }
  } else {
    switch (key) {
      case 111: VA_LAUNCH(1, 1, 1);
      case 112: VA_LAUNCH(1, 1, 2);
      case 114: VA_LAUNCH(1, 1, 4);
      case 211: VA_LAUNCH(2, 1, 1);
      case 212: VA_LAUNCH(2, 1, 2);
      case 214: VA_LAUNCH(2, 1, 4);
      case 221: VA_LAUNCH(2, 2, 1);
      case 222: VA_LAUNCH(2, 2, 2);
      case 241: VA_LAUNCH(2, 4, 1);
      default: return VA_EUNSUPPORTED;
    }
  }
#undef VA_LAUNCH
}

}  // namespace

int launch_splitkv_fwd(const verify_attn_args* a, const Plan& p, hipStream_t st) {
  if (a->batch > 65535 || a->hkv > 65535) return VA_EUNSUPPORTED;
  const int eb = a->kv_dtype == VA_KV_FP8_E4M3FN ? 1 : 2;
  FwdParams fp;
  fp.q = static_cast<const uint8_t*>(a->q);
  fp.q_srow = a->q_stride_row * 2;
  fp.q_shead = a->q_stride_head * 2;
  fp.k = static_cast<const uint8_t*>(a->k_cache);
  fp.k_sslot = a->k_stride_slot * eb;
  fp.k_shead = a->k_stride_head * eb;
  fp.v = static_cast<const uint8_t*>(a->v_cache);
  fp.v_sslot = a->v_stride_slot * eb;
  fp.v_shead = a->v_stride_head * eb;
  fp.bt = a->block_table;
  fp.max_pages = a->max_pages_per_seq;
  fp.prefix_lens = a->prefix_lens;
  fp.part_o = a->workspace;
  fp.part_lse = a->workspace + p.ws_o_floats;
  fp.counts = reinterpret_cast<int32_t*>(a->workspace + p.ws_cnt_floats);
  fp.batch = a->batch;
  fp.hkv = a->hkv;
  fp.group = p.group;
  fp.draft = a->draft_len;
  fp.rows = p.rows;
  fp.lg_page = p.lg_page;
  fp.window = a->window_left;
  fp.slots = p.slots;
  fp.min_q = p.min_q;
  fp.piece_cost = p.piece_cost;
  fp.c_log2 = a->sm_scale * a->k_scale * kLog2e;
  fp.v_scale = a->v_scale;
  fp.qo_indptr = a->qo_indptr;
  fp.draft_slots = a->draft_slots;
  fp.tree_mask = a->tree_mask;
  fp.logit_cap = a->logit_cap;
  // grid: x = head groups (fastest, so the heads of one key range are read together),
  // y = key ranges of the balanced partition
  const dim3 grid(p.hg, p.nwy, 1);
  if (p.kind == kMlaFp8) return launch_splitkv_mla_fp8(fp, p, grid, st);
  if (p.kind == kTile) return launch_splitkv_tile(fp, a->qk_dim, p.hpc, p.nrg, grid, st);
  const bool f8 = a->kv_dtype == VA_KV_FP8_E4M3FN;
  const bool ext = a->draft_slots != nullptr || a->logit_cap > 0.f;
#define VA_DIMS(DK_, DV_)                                                                   \
  return f8 ? (ext ? launch_dims<DK_, DV_, true, true>(fp, p, grid, st)                      \
                   : launch_dims<DK_, DV_, true, false>(fp, p, grid, st))                    \
            : (ext ? launch_dims<DK_, DV_, false, true>(fp, p, grid, st)                     \
                   : launch_dims<DK_, DV_, false, false>(fp, p, grid, st))
  if (a->qk_dim == 128) VA_DIMS(128, 128);
  if (a->qk_dim == 256) VA_DIMS(256, 256);
  if (a->qk_dim == 576) VA_DIMS(576, 512);
#undef VA_DIMS
  return VA_EUNSUPPORTED;
}

}  // namespace va
