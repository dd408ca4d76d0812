// Combine stage of split-KV target verify (PR #27382, "Modifications": the second
// stage merges the per-split partials by log-sum-exp).
//
// The split-KV pass already covered every key of a row, the causal draft keys
// included, in a sequence's pieces; the combine merges the pieces' (O, LSE)
// partials.  One wave per query row (draft i, q head h), lanes across the row's
// columns; a workgroup holds 4 rows of one (sequence b, KV head g).  Per row:
//   M = max of the pieces' LSEs, weights e^{LSE - M} (a piece in which the row
//   sees no key has LSE = -inf and weight 0), out = weighted mean in bf16 (round
//   to nearest even), lse = M + log(sum of weights).  An attention sink is one
//   more term with LSE = the sink logit and a zero output (the split-KV page's
//   can_handle() lists sinks among what its fast path does not serve).
// Every row sees at least its own draft key, so M and the final LSE are finite.

#include <math.h>

#include "va_internal.h"

namespace va {

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* counts;
  uint16_t* out;
  int64_t o_srow, o_shead;   // elements
  float* lse;
  int hkv, group, draft, rows, slots;
  const int32_t* qo_indptr;  // ragged rows, or NULL (row b*D + i)
  const float* sinks;        // [hq] sink logits, or NULL
};

namespace {

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

// CPT consecutive floats of one partial row.
template <int CPT>
struct Cols {
  float v[CPT];
};

template <int CPT>
__device__ __forceinline__ Cols<CPT> load_cols(const float* p) {
  Cols<CPT> c;
  if constexpr (CPT % 4 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; k += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(p + k);
      c.v[k] = x[0];
      c.v[k + 1] = x[1];
      c.v[k + 2] = x[2];
      c.v[k + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) c.v[k] = p[k];
  }
  return c;
}

}  // namespace

template <int DV>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams P) {
  constexpr int CPT = DV / 64;  // output columns per lane
  constexpr bool kReuse = DV >= 512;
  constexpr int NB = kReuse ? 12 : 8;  // partial rows loaded per batch
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (row >= P.rows) return;  // no barriers in this kernel
  const int i = row / P.group;
  const int nrow_b = P.qo_indptr ? P.qo_indptr[b + 1] - P.qo_indptr[b] : P.draft;
  if (i >= nrow_b) return;    // the sequence has fewer draft rows (draft-extend)
  const int h = g * P.group + row % P.group;
  const int r = (P.qo_indptr ? P.qo_indptr[b] : b * P.draft) + i;

  int n = P.counts[b];
  n = n < 1 ? 1 : (n > P.slots ? P.slots : n);
  const int64_t split0 = ((int64_t)b * P.hkv + g) * P.slots;
  const float* plse = P.part_lse + split0 * P.rows + row;
  const float* po = P.part_o + (split0 * P.rows + row) * DV + lane * CPT;
  const int64_t pstride = (int64_t)P.rows * DV;

  // lane s holds piece s's LSE (64 pieces per pass); the first NB pieces' columns
  // are loaded alongside, so one round trip serves the common case.  Wide rows
  // (v_dim 512) reuse one register buffer for every batch, which keeps the kernel
  // under 128 registers; narrower rows load each later batch into fresh registers.
  Cols<CPT> first[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u)
    if (u < n) first[u] = load_cols<CPT>(po + u * pstride);
  // a sink joins the denominator as one more partial with a zero output
  const float sink = P.sinks ? P.sinks[h] : -INFINITY;
  float M = sink;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const float ls = (s0 + lane < n) ? plse[(int64_t)(s0 + lane) * P.rows] : -INFINITY;
    M = fmaxf(M, wave_max(ls));
  }

  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
  float Z = sink == -INFINITY ? 0.f : expf(sink - M);
  for (int s0 = 0; s0 < n; s0 += 64) {
    const float ls = (s0 + lane < n) ? plse[(int64_t)(s0 + lane) * P.rows] : -INFINITY;
    const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);
    Z += wave_sum(w);
    const int cnt = min(64, n - s0);
    for (int s = 0; s < cnt; s += NB) {
      if constexpr (kReuse) {
        if (s0 > 0 || s > 0) {
#pragma unroll
          for (int u = 0; u < NB; ++u)
            if (s + u < cnt) first[u] = load_cols<CPT>(po + (int64_t)(s0 + s + u) * pstride);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (s + u >= cnt) break;
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s + u));
#pragma unroll
          for (int c = 0; c < CPT; ++c) acc[c] += wu * first[u].v[c];
        }
      } else {
        Cols<CPT> vals[NB];
        if (s0 == 0 && s == 0) {
#pragma unroll
          for (int u = 0; u < NB; ++u) vals[u] = first[u];
        } else {
#pragma unroll
          for (int u = 0; u < NB; ++u)
            if (s + u < cnt) vals[u] = load_cols<CPT>(po + (int64_t)(s0 + s + u) * pstride);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (s + u >= cnt) break;
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s + u));
#pragma unroll
          for (int c = 0; c < CPT; ++c) acc[c] += wu * vals[u].v[c];
        }
      }
    }
  }
  const float invZ = 1.f / Z;
  uint16_t* op = P.out + (int64_t)r * P.o_srow + (int64_t)h * P.o_shead + lane * CPT;
#pragma unroll
  for (int c = 0; c < CPT; ++c) op[c] = f32_to_bf16_rne(acc[c] * invZ);
  if (P.lse && lane == 0) P.lse[(int64_t)r * (P.hkv * P.group) + h] = M + logf(Z);
}

// Rows whose sequence may span many pieces (the slot count is large when few
// sequences spread over the whole chip): W waves share one row, wave w merging pieces
// w, w + W, w + 2W, ... against its own maximum, so W times as many partial rows are
// in flight; wave 0 then merges the W results through LDS.  One row per workgroup,
// so every wave takes the same exits and all of them reach the one barrier.
template <int DV, int W>
__global__ __launch_bounds__(64 * W) void combine_split_kernel(CombineParams P) {
  constexpr int CPT = DV / 64;  // output columns per lane
  constexpr int NB = 8;         // partial rows in flight per wave
  __shared__ float s_acc[W][DV];
  __shared__ float s_mz[W][2];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int row = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (row >= P.rows) return;
  const int i = row / P.group;
  const int nrow_b = P.qo_indptr ? P.qo_indptr[b + 1] - P.qo_indptr[b] : P.draft;
  if (i >= nrow_b) return;
  const int h = g * P.group + row % P.group;
  const int r = (P.qo_indptr ? P.qo_indptr[b] : b * P.draft) + i;

  int n = P.counts[b];
  n = n < 1 ? 1 : (n > P.slots ? P.slots : n);
  const int64_t split0 = ((int64_t)b * P.hkv + g) * P.slots;
  const float* plse = P.part_lse + split0 * P.rows + row;
  const float* po = P.part_o + (split0 * P.rows + row) * DV + lane * CPT;
  const int64_t pstride = (int64_t)P.rows * DV;
  const int nw = n > w ? (n - w + W - 1) / W : 0;  // this wave's pieces

  float Mw = -INFINITY;
  for (int t0 = 0; t0 < nw; t0 += 64) {
    const float ls = (t0 + lane < nw) ? plse[(int64_t)(w + W * (t0 + lane)) * P.rows] : -INFINITY;
    Mw = fmaxf(Mw, wave_max(ls));
  }
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
  float Zw = 0.f;
  for (int t0 = 0; t0 < nw; t0 += 64) {
    const float ls = (t0 + lane < nw) ? plse[(int64_t)(w + W * (t0 + lane)) * P.rows] : -INFINITY;
    const float wt = (ls == -INFINITY) ? 0.f : expf(ls - Mw);
    Zw += wave_sum(wt);
    const int cnt = min(64, nw - t0);
    for (int s = 0; s < cnt; s += NB) {
      Cols<CPT> vals[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (s + u < cnt) vals[u] = load_cols<CPT>(po + (int64_t)(w + W * (t0 + s + u)) * pstride);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (s + u >= cnt) break;
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), s + u));
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] += wu * vals[u].v[c];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) s_acc[w][lane * CPT + c] = acc[c];
  if (lane == 0) {
    s_mz[w][0] = Mw;
    s_mz[w][1] = Zw;
  }
  __syncthreads();
  if (w != 0) return;
  // a sink joins the denominator as one more partial with a zero output
  const float sink = P.sinks ? P.sinks[h] : -INFINITY;
  float M = sink;
#pragma unroll
  for (int v = 0; v < W; ++v) M = fmaxf(M, s_mz[v][0]);
  float Z = sink == -INFINITY ? 0.f : expf(sink - M);
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
  // (unrolled by 4: a full unroll would hold all W waves' columns in registers at once)
#pragma unroll 4
  for (int v = 0; v < W; ++v) {
    const float f = s_mz[v][0] == -INFINITY ? 0.f : expf(s_mz[v][0] - M);
    Z += f * s_mz[v][1];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] += f * s_acc[v][lane * CPT + c];
  }
  const float invZ = 1.f / Z;
  uint16_t* op = P.out + (int64_t)r * P.o_srow + (int64_t)h * P.o_shead + lane * CPT;
#pragma unroll
  for (int c = 0; c < CPT; ++c) op[c] = f32_to_bf16_rne(acc[c] * invZ);
  if (P.lse && lane == 0) P.lse[(int64_t)r * (P.hkv * P.group) + h] = M + logf(Z);
}

int launch_combine(const verify_attn_args* a, const Plan& p, hipStream_t st) {
  if (a->batch > 65535 || a->hkv > 65535) return VA_EUNSUPPORTED;
  CombineParams cp;
  cp.part_o = a->workspace;
  cp.part_lse = a->workspace + p.ws_o_floats;
  cp.counts = reinterpret_cast<const int32_t*>(a->workspace + p.ws_cnt_floats);
  cp.out = static_cast<uint16_t*>(a->out);
  cp.o_srow = a->o_stride_row;
  cp.o_shead = a->o_stride_head;
  cp.lse = a->lse;
  cp.hkv = a->hkv;
  cp.group = p.group;
  cp.draft = a->draft_len;
  cp.rows = p.rows;
  cp.slots = p.slots;
  cp.qo_indptr = a->qo_indptr;
  cp.sinks = a->sinks;
  // up to 32 slots: one wave per row; more: 4 or 16 waves share a row, while the grid
  // stays within 16 waves per CU.  Thousands of rows fill the chip with one wave each,
  // and there the extra waves' merge through LDS only costs time (a row's count is at
  // most the split pass's grid height over the batch, so many rows also mean few pieces)
  const int64_t nrows = (int64_t)a->batch * a->hkv * p.rows;
  int wpr = p.slots > 64 ? 16 : (p.slots > 32 ? 4 : 1);
  while (wpr > 1 && nrows * wpr > 16LL * device_cu_count()) wpr /= 4;
  if (wpr == 1) {
    const dim3 grid((p.rows + kWaves - 1) / kWaves, a->hkv, a->batch);
#define VA_LAUNCH(DV_) \
    return launch_kernel(reinterpret_cast<const void*>(&combine_kernel<DV_>), grid, dim3(256), cp, st)
    if (a->v_dim == 128) VA_LAUNCH(128);
    if (a->v_dim == 256) VA_LAUNCH(256);
    if (a->v_dim == 512) VA_LAUNCH(512);
#undef VA_LAUNCH
    return VA_EUNSUPPORTED;
  }
  const dim3 grid(p.rows, a->hkv, a->batch);
#define VA_LAUNCH(DV_, W_)                                                                     \
  return launch_kernel(reinterpret_cast<const void*>(&combine_split_kernel<DV_, W_>), grid, \
                       dim3(64 * (W_)), cp, st)
  if (wpr == 4) {
    if (a->v_dim == 128) VA_LAUNCH(128, 4);
    if (a->v_dim == 256) VA_LAUNCH(256, 4);
    if (a->v_dim == 512) VA_LAUNCH(512, 4);
  } else {
    if (a->v_dim == 128) VA_LAUNCH(128, 16);
    if (a->v_dim == 256) VA_LAUNCH(256, 16);
    if (a->v_dim == 512) VA_LAUNCH(512, 16);
  }
#undef VA_LAUNCH
  return VA_EUNSUPPORTED;
}

}  // namespace va
