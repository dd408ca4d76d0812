// Split-KV (flash-decode) pass over the prefix for EAGLE target-verify at topk = 1.
//
// PR #27382 ("[AMD][Perf] Split-KV flash-decode attention for EAGLE target-verify",
// sections "Motivation" and "Modifications") splits the long shared prefix across
// parallel programs, each writing a partial output and log-sum-exp that a second
// stage merges.  This is the gfx950 design of that first stage:
//
//   workgroup = (split s, KV head g, sequence b), 4 waves of 64 lanes.
//   All G*D query rows of KV head g form the dense M dimension (16/32/64 rows).
//   The rows are cut into NRG row groups of 16*RT rows; the 4/NRG waves of a row
//   group interleave the split's 32-token blocks.
//
// Per 32-token block a wave
//   1. maps each token to its slot through the block table (page = bt[t >> lgP]),
//   2. loads K rows straight into MFMA A-operand registers (lane l: token l%16,
//      16 contiguous bytes of the row; four lanes cover 64 B of one row),
//   3. loads V rows coalesced (16 lanes read one full row) for 8 tokens per lane,
//   4. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp8 K is widened to
//      bf16 exactly in registers), so each lane ends up with 8 scores of ONE row,
//   5. runs the online softmax in the exp2 domain (row max across the 4 lanes
//      of a row by two xor-shuffles, running sum kept per lane),
//   6. computes O^T += V^T P^T: the lane's own 8 probabilities are the B operand
//      (no data movement), and V^T's A operand is an 8x8 transpose done inside
//      the lane's registers (the column permutation is undone on the write).
// The waves of a row group then merge through LDS in a fixed order (bitwise
// deterministic) and the last one writes the split's partial O (normalised,
// times v_scale) and LSE (natural log) to the workspace.
//
// Masking: the tail of a split and, with a left window W, keys t < L + i - W of
// row i.  Masked scores are set to -inf by selection; masked token loads are
// clamped to the split's last real token so no load leaves the sequence.

#include <limits.h>
#include <math.h>

#include "va_internal.h"

namespace va {

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

template <int NB>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* dst) {
  if constexpr (NB == 8) {
    u32x2 v = *reinterpret_cast<const u32x2*>(p);
    dst[0] = v[0];
    dst[1] = v[1];
  } else {
#pragma unroll
    for (int c = 0; c < NB / 16; ++c) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * c);
      dst[4 * c + 0] = v[0];
      dst[4 * c + 1] = v[1];
      dst[4 * c + 2] = v[2];
      dst[4 * c + 3] = v[3];
    }
  }
}

// Token position of slot i (0..7) of lane group j inside a 32-token block.  The
// S^T accumulator of token tile tt holds tokens 16*tt + 4*j + r (r = 0..3) in a
// lane, so slots 0..3 are tile 0 and slots 4..7 tile 1.  P^T and V^T use the same
// order, which is all the MFMA reduction needs.
__device__ __forceinline__ int slot_token(int j, int i) {
  return (i < 4) ? (4 * j + i) : (16 + 4 * j + (i - 4));
}

__device__ __forceinline__ int64_t token_slot(const int32_t* bt_row, int t, int lg, int pmask) {
  const int page = bt_row[t >> lg];
  return ((int64_t)page << lg) | (int64_t)(t & pmask);
}

}  // namespace

template <int DK, int DV, bool FP8, int RT, int NRG>
__global__ __launch_bounds__(256) void splitkv_fwd_kernel(FwdParams P) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KSTEPS = DK / 32;          // MFMA k-steps over qk_dim
  constexpr int KLOADS = DK * EB / 64;     // 16-B K loads per lane per token tile
  constexpr int CPL = DV / 16;             // V columns per lane per token (= O^T col tiles)
  constexpr int VBYTES = CPL * EB;
  constexpr int VW = VBYTES / 4;
  constexpr int NTL = kWaves / NRG;        // waves sharing one row group
  static_assert(DK % 64 == 0 || !FP8, "fp8 K loads cover two k-steps");
  static_assert(VBYTES == 8 || VBYTES % 16 == 0, "V chunk");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int rg = wave % NRG;
  const int tl = wave / NRG;
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  // a2: this split's slice of the attended prefix [lo, L)
  const int L = P.prefix_lens[b];
  const int lo = P.window >= 0 ? max(0, L - P.window) : 0;
  const int nsplit = (L - lo + P.chunk - 1) / P.chunk;
  if (s >= nsplit) return;  // uniform over the workgroup, before any barrier
  const int t_begin = lo + s * P.chunk;
  const int t_end = (s == P.splits - 1) ? L : min(L, t_begin + P.chunk);
  const int nblk = (t_end - t_begin + kTokBlock - 1) / kTokBlock;

  // Q^T as the B operand: lane holds row n of each row tile, 8 consecutive k-slots.
  bf16x8 qB[RT][KSTEPS];
  int row_lo[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (rg * RT + rt) * 16 + n;
    const bool rv = row < P.rows;
    const int i = rv ? row / P.group : 0;
    const int hh = rv ? row % P.group : 0;
    row_lo[rt] = P.window >= 0 ? L + i - P.window : INT_MIN;
    const uint8_t* qp =
        P.q + (int64_t)(b * P.draft + i) * P.q_srow + (int64_t)(g * P.group + hh) * P.q_shead;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      // element offset of this lane's 8 k-slots; must match the K operand below
      const int d0 = FP8 ? (64 * (ks / 2) + 16 * j + 8 * (ks % 2)) : (32 * ks + 8 * j);
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (rv) raw = *reinterpret_cast<const u32x4*>(qp + 2 * d0);
      qB[rt][ks] = as_bf16x8(raw);
    }
  }

  float m_run[RT], l_run[RT];
  f32x4 oacc[RT][CPL];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) oacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;
  const uint8_t* kbase = P.k + (int64_t)g * P.k_shead + 16 * j;
  const uint8_t* vbase = P.v + (int64_t)g * P.v_shead + n * VBYTES;
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;

  for (int blk = tl; blk < nblk; blk += NTL) {
    const int t0 = t_begin + blk * kTokBlock;

    // a3: gather.  K: token 16*tt + n of the block.  V: the lane's 8 slot tokens.
    u32x4 kraw[2][KLOADS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = min(t0 + 16 * tt + n, t_end - 1);
      const uint8_t* kp = kbase + token_slot(bt_row, t, lg, pmask) * P.k_sslot;
#pragma unroll
      for (int u = 0; u < KLOADS; ++u) kraw[tt][u] = *reinterpret_cast<const u32x4*>(kp + 64 * u);
    }
    uint32_t vraw[8][VW];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = min(t0 + slot_token(j, e), t_end - 1);
      load_bytes<VBYTES>(vbase + token_slot(bt_row, t, lg, pmask) * P.v_sslot, vraw[e]);
    }

    // a4: S^T = K Q^T
    f32x4 sacc[2][RT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sacc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 a;
        if constexpr (FP8) {
          const u32x4 c = kraw[tt][ks / 2];
          const u32x2 w0 = fp8x4_to_bf16x4(c[2 * (ks % 2)]);
          const u32x2 w1 = fp8x4_to_bf16x4(c[2 * (ks % 2) + 1]);
          a = as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]});
        } else {
          a = as_bf16x8(kraw[tt][ks]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[rt][ks], sacc[tt][rt], 0, 0, 0);
      }
    }

    // online softmax (exp2 domain); lane holds 8 scores of row n of each row tile
    bf16x8 pB[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sc[8];
      float bmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = e >> 2, r = e & 3;
        const int t = t0 + 16 * tt + 4 * j + r;
        const bool ok = (t < t_end) && (t >= row_lo[rt]);
        const float v = ok ? sacc[tt][rt][r] * P.c_log2 : -INFINITY;
        sc[e] = v;
        bmax = fmaxf(bmax, v);
      }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float m_new = fmaxf(m_run[rt], bmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sc[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
        psum += sc[e];
      }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int ct = 0; ct < CPL; ++ct) oacc[rt][ct] *= alpha;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[e];
      pB[rt] = pb;
    }

    // a5: O^T += V^T P^T.  Column tile ct holds column CPL*m + ct in row m.
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) {
      u32x4 av;
      if constexpr (FP8) {
        const int w = ct >> 2, sh = 8 * (ct & 3);
        uint32_t x0 = 0, x1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x0 |= ((vraw[e][w] >> sh) & 0xffu) << (8 * e);
          x1 |= ((vraw[4 + e][w] >> sh) & 0xffu) << (8 * e);
        }
        const u32x2 c0 = fp8x4_to_bf16x4(x0);
        const u32x2 c1 = fp8x4_to_bf16x4(x1);
        av = u32x4{c0[0], c0[1], c1[0], c1[1]};
      } else {
        const int w = ct >> 1;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t a0 = vraw[2 * q2][w], a1 = vraw[2 * q2 + 1][w];
          av[q2] = (ct & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
      }
      const bf16x8 a = as_bf16x8(av);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        oacc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB[rt], oacc[rt][ct], 0, 0, 0);
    }
  }

  // each lane summed only its own tokens: total the 4 lanes of a row
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16, 64);
    l_run[rt] += __shfl_xor(l_run[rt], 32, 64);
  }

  if constexpr (NTL > 1) {
    // merge the waves of each row group in a fixed order through LDS
    constexpr int NREG = RT * CPL * 4 + RT;
    __shared__ float sm_m[kWaves][RT][16];
    __shared__ float sm_o[NRG][NREG][64];
    if (j == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sm_m[wave][rt][n] = m_run[rt];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < NTL; ++k) M = fmaxf(M, sm_m[k * NRG + rg][rt][n]);
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
              for (int r = 0; r < 4; ++r) oacc[rt][ct][r] += sm_o[rg][(rt * CPL + ct) * 4 + r][lane];
            l_run[rt] += sm_o[rg][RT * CPL * 4 + rt][lane];
          }
        }
        if (k < NTL - 1) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
              for (int r = 0; r < 4; ++r) sm_o[rg][(rt * CPL + ct) * 4 + r][lane] = oacc[rt][ct][r];
            sm_o[rg][RT * CPL * 4 + rt][lane] = l_run[rt];
          }
        }
      }
      __syncthreads();
    }
    if (tl != NTL - 1) return;
  }

  // write the split's partial: lane holds row n, columns [4*CPL*j, 4*CPL*(j+1))
  const int64_t split_id = ((int64_t)b * P.hkv + g) * P.splits + s;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (rg * RT + rt) * 16 + n;
    if (row >= P.rows) continue;
    const float l = l_run[rt];
    const float inv = l > 0.f ? P.v_scale / l : 0.f;
    float* po = P.part_o + (split_id * P.rows + row) * DV + 4 * CPL * j;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int c4 = 0; c4 < CPL; c4 += 4) {
        f32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = oacc[rt][c4 + c][r] * inv;
        *reinterpret_cast<f32x4*>(po + CPL * r + c4) = o;
      }
    }
    if (j == 0)
      P.part_lse[split_id * P.rows + row] = l > 0.f ? (m_run[rt] + log2f(l)) * kLn2 : -INFINITY;
  }
}

namespace {

template <int DK, int DV, bool FP8>
int launch_dims(const FwdParams& fp, const Plan& p, dim3 grid, hipStream_t st) {
#define VA_LAUNCH(RT_, NRG_) \
  hipLaunchKernelGGL((splitkv_fwd_kernel<DK, DV, FP8, RT_, NRG_>), grid, dim3(256), 0, st, fp)
  if constexpr (DV > 256) {
    // a 512-wide O^T already fills 128 accumulator registers: one row tile per wave
    if (p.rt == 1 && p.nrg == 1) VA_LAUNCH(1, 1);
    else if (p.rt == 1 && p.nrg == 2) VA_LAUNCH(1, 2);
    else if (p.rt == 1 && p.nrg == 4) VA_LAUNCH(1, 4);
    else return VA_EUNSUPPORTED;
  } else {
    if (p.rt == 1 && p.nrg == 1) VA_LAUNCH(1, 1);
    else if (p.rt == 2 && p.nrg == 1) VA_LAUNCH(2, 1);
    else if (p.rt == 2 && p.nrg == 2) VA_LAUNCH(2, 2);
    else if (p.rt == 2 && p.nrg == 4) VA_LAUNCH(2, 4);
    else return VA_EUNSUPPORTED;
  }
#undef VA_LAUNCH
  return hipGetLastError() == hipSuccess ? VA_OK : VA_EHIP;
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
  fp.hkv = a->hkv;
  fp.group = p.group;
  fp.draft = a->draft_len;
  fp.rows = p.rows;
  fp.lg_page = p.lg_page;
  fp.window = a->window_left;
  fp.splits = p.splits;
  fp.chunk = p.chunk;
  fp.c_log2 = a->sm_scale * a->k_scale * kLog2e;
  fp.v_scale = a->v_scale;
  const dim3 grid(p.splits, a->hkv, a->batch);
  const bool f8 = a->kv_dtype == VA_KV_FP8_E4M3FN;
  if (a->qk_dim == 128) return f8 ? launch_dims<128, 128, true>(fp, p, grid, st)
                                  : launch_dims<128, 128, false>(fp, p, grid, st);
  if (a->qk_dim == 256) return f8 ? launch_dims<256, 256, true>(fp, p, grid, st)
                                  : launch_dims<256, 256, false>(fp, p, grid, st);
  if (a->qk_dim == 576) return f8 ? launch_dims<576, 512, true>(fp, p, grid, st)
                                  : launch_dims<576, 512, false>(fp, p, grid, st);
  return VA_EUNSUPPORTED;
}

}  // namespace va
