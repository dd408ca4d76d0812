// Combine stage of split-KV target verify (PR #27382, "Modifications": the second
// stage merges the prefix splits by log-sum-exp and adds the small causal
// draft-draft block).
//
// One wave per query row (draft i, q head h), lanes across the row's columns; a
// workgroup holds 4 rows of one (sequence b, KV head g).  Per row:
//   draft block: keys L+j for j <= i (and j >= i - W with a left window W), scores
//   in fp32 from the bf16 q and the (dequantised) cached draft keys, softmax over
//   them -> one more (O, LSE) partial;
//   merge: M = max LSE over the used splits and the draft partial, weights
//   e^{LSE - M} (an empty split has LSE = -inf and weight 0), out = weighted mean in
//   bf16 (round to nearest even), lse = M + log(sum of weights).
// Every row sees at least itself, so the final LSE is finite.

#include <math.h>

#include "va_internal.h"

namespace va {

struct CombineParams {
  const uint8_t* q;
  int64_t q_srow, q_shead;   // bytes
  const uint8_t* k;
  int64_t k_sslot, k_shead;  // bytes
  const uint8_t* v;
  int64_t v_sslot, v_shead;  // bytes
  const int32_t* bt;
  int32_t max_pages;
  const int32_t* prefix_lens;
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  int64_t o_srow, o_shead;   // elements
  float* lse;
  int hkv, group, draft, rows, lg_page, window, splits, chunk;
  float c_nat;  // sm_scale * k_scale
  float v_scale;
};

namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// OCP fp8 e4m3fn -> float from the bit layout (sign, 4-bit exponent bias 7, 3-bit
// mantissa; exponent 0 = subnormal m/8 * 2^-6; S.1111.111 = NaN).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  float mag;
  if (e == 0xfu && m == 7u) mag = __uint_as_float(0x7fc00000u);
  else if (e == 0) mag = (float)m * 0.001953125f;  // m * 2^-9
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

template <bool FP8>
__device__ __forceinline__ float load_elem(const uint8_t* row, int idx) {
  if constexpr (FP8) return e4m3fn_to_f32(row[idx]);
  else return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[idx]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

}  // namespace

// One wave per query row (draft i, q head h of KV head g, sequence b); lanes span
// the row's columns.  Workgroup = 4 consecutive rows of one (b, g).
template <int DK, int DV, bool FP8>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams P) {
  constexpr int DPL = DK / 64;  // q/k elements per lane in a dot product
  constexpr int CPT = DV / 64;  // output columns per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (row >= P.rows) return;  // no barriers in this kernel

  const int L = P.prefix_lens[b];
  const int lo = P.window >= 0 ? max(0, L - P.window) : 0;
  int nsplit = (L - lo + P.chunk - 1) / P.chunk;
  if (nsplit > P.splits) nsplit = P.splits;  // the last split absorbed the rest
  const int32_t* bt_row = P.bt + (int64_t)b * P.max_pages;
  const int lg = P.lg_page;
  const int pmask = (1 << lg) - 1;
  const int i = row / P.group;
  const int h = g * P.group + row % P.group;
  const int r = b * P.draft + i;
  const int64_t split0 = ((int64_t)b * P.hkv + g) * P.splits;

  // a6: draft-draft block, keys L+jj for jj <= i inside the window (never empty)
  float qv[DPL];
  const uint16_t* qp =
      reinterpret_cast<const uint16_t*>(P.q + (int64_t)r * P.q_srow + (int64_t)h * P.q_shead);
#pragma unroll
  for (int k = 0; k < DPL; ++k) qv[k] = bf16_bits_to_f32(qp[lane * DPL + k]);
  const int jlo = P.window >= 0 ? max(0, i - P.window) : 0;
  float sc[8];
  const uint8_t* vrow[8];
  float mx = -INFINITY;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    sc[jj] = -INFINITY;
    vrow[jj] = nullptr;
    if (jj < jlo || jj > i) continue;
    const int t = L + jj;
    const int64_t slot = ((int64_t)bt_row[t >> lg] << lg) | (int64_t)(t & pmask);
    const uint8_t* kr = P.k + slot * P.k_sslot + (int64_t)g * P.k_shead;
    vrow[jj] = P.v + slot * P.v_sslot + (int64_t)g * P.v_shead;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc += qv[k] * load_elem<FP8>(kr, lane * DPL + k);
    sc[jj] = wave_sum(acc) * P.c_nat;
    mx = fmaxf(mx, sc[jj]);
  }
  float od[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) od[c] = 0.f;
  float zd = 0.f;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    if (vrow[jj] == nullptr) continue;
    const float w = expf(sc[jj] - mx);
    zd += w;
#pragma unroll
    for (int c = 0; c < CPT; ++c) od[c] += w * load_elem<FP8>(vrow[jj], lane * CPT + c);
  }
  const float lse_d = mx + logf(zd);

  // a7: log-sum-exp merge.  Lane s holds split s's LSE (64 splits per pass).
  const float* plse = P.part_lse + split0 * P.rows + row;
  float M = lse_d;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const float ls = (s0 + lane < nsplit) ? plse[(int64_t)(s0 + lane) * P.rows] : -INFINITY;
    M = fmaxf(M, wave_max(ls));
  }
  const float wd = expf(lse_d - M);
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = wd * od[c] * (P.v_scale / zd);
  float Z = wd;
  const float* po = P.part_o + (split0 * P.rows + row) * DV + lane * CPT;
  const int64_t pstride = (int64_t)P.rows * DV;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const float ls = (s0 + lane < nsplit) ? plse[(int64_t)(s0 + lane) * P.rows] : -INFINITY;
    const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);
    Z += wave_sum(w);
    const int cnt = min(64, nsplit - s0);
    int s = 0;
    for (; s + 4 <= cnt; s += 4) {
      float ws[4];
      float vals[4][CPT];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ws[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s + u));
        const float* p = po + (int64_t)(s0 + s + u) * pstride;
#pragma unroll
        for (int c = 0; c < CPT; ++c) vals[u][c] = p[c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] += ws[u] * vals[u][c];
      }
    }
    for (; s < cnt; ++s) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
      const float* p = po + (int64_t)(s0 + s) * pstride;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] += wu * p[c];
    }
  }
  const float invZ = 1.f / Z;
  uint16_t* op = P.out + (int64_t)r * P.o_srow + (int64_t)h * P.o_shead + lane * CPT;
#pragma unroll
  for (int c = 0; c < CPT; ++c) op[c] = f32_to_bf16_rne(acc[c] * invZ);
  if (P.lse && lane == 0) P.lse[(int64_t)r * (P.hkv * P.group) + h] = M + logf(Z);
}

int launch_combine(const verify_attn_args* a, const Plan& p, hipStream_t st) {
  if (a->batch > 65535 || a->hkv > 65535) return VA_EUNSUPPORTED;
  const int eb = a->kv_dtype == VA_KV_FP8_E4M3FN ? 1 : 2;
  CombineParams cp;
  cp.q = static_cast<const uint8_t*>(a->q);
  cp.q_srow = a->q_stride_row * 2;
  cp.q_shead = a->q_stride_head * 2;
  cp.k = static_cast<const uint8_t*>(a->k_cache);
  cp.k_sslot = a->k_stride_slot * eb;
  cp.k_shead = a->k_stride_head * eb;
  cp.v = static_cast<const uint8_t*>(a->v_cache);
  cp.v_sslot = a->v_stride_slot * eb;
  cp.v_shead = a->v_stride_head * eb;
  cp.bt = a->block_table;
  cp.max_pages = a->max_pages_per_seq;
  cp.prefix_lens = a->prefix_lens;
  cp.part_o = a->workspace;
  cp.part_lse = a->workspace + p.ws_o_floats;
  cp.out = static_cast<uint16_t*>(a->out);
  cp.o_srow = a->o_stride_row;
  cp.o_shead = a->o_stride_head;
  cp.lse = a->lse;
  cp.hkv = a->hkv;
  cp.group = p.group;
  cp.draft = a->draft_len;
  cp.rows = p.rows;
  cp.lg_page = p.lg_page;
  cp.window = a->window_left;
  cp.splits = p.splits;
  cp.chunk = p.chunk;
  cp.c_nat = a->sm_scale * a->k_scale;
  cp.v_scale = a->v_scale;
  const dim3 grid((p.rows + kWaves - 1) / kWaves, a->hkv, a->batch);
  const bool f8 = a->kv_dtype == VA_KV_FP8_E4M3FN;
#define VA_LAUNCH(DK_, DV_, F8_) \
  return launch_kernel(reinterpret_cast<const void*>(&combine_kernel<DK_, DV_, F8_>), grid, \
                       dim3(256), cp, st)
  if (a->qk_dim == 128) { if (f8) VA_LAUNCH(128, 128, true); else VA_LAUNCH(128, 128, false); }
  else if (a->qk_dim == 256) { if (f8) VA_LAUNCH(256, 256, true); else VA_LAUNCH(256, 256, false); }
  else if (a->qk_dim == 576) { if (f8) VA_LAUNCH(576, 512, true); else VA_LAUNCH(576, 512, false); }
#undef VA_LAUNCH
  return VA_EUNSUPPORTED;
}

}  // namespace va
