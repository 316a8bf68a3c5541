// Accepted-path state reconstruction (paper Eq. 10; review: one batched commit
// over all recurrent layers), in place on the state pool:
//
//   S[v][c] <- P_a S[v][c] + sum_{j in path(a)} (P_a/P_j) U_j[v] k_j[c]
//
// One workgroup per (layer, request, head).  The path sum is a
// [d_v x L_a] x [L_a x d_k] product on bf16 MFMA (K = path position, padded to
// 32): A = (P_a/P_j) U_j (float32, split hi+lo), B = k_j (bf16 exact; float32
// keys are split as well).  The P_a S term is applied in float32 in the
// epilogue, so every slot element is read once and written once.
#include "common.h"

namespace bole {

template <int DT>
__device__ __forceinline__ void load_key8(const void* k, int64_t row_stride_elems,
                                          const int* pj, int p0, int La, int64_t base, int c,
                                          bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int p = p0 + e;
    float val = 0.0f;
    if (p < La) {
      const int64_t idx = base + (int64_t)pj[p] * row_stride_elems + c;
      if (DT == BOLE_BF16)
        val = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(k)[idx]);
      else
        val = reinterpret_cast<const float*>(k)[idx];
    }
    x[e] = val;
  }
  if (DT == BOLE_BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) hi[e] = (__bf16)x[e];  // exact: values are bf16
    lo = zero_bf16x8();
  } else {
    split_bf16x8(x, hi, lo);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void commit_kernel(
    float* __restrict__ state_pool, int64_t state_layer_stride, int32_t n_slots,
    const int32_t* __restrict__ slot, const void* __restrict__ kmat, int64_t k_layer_stride,
    const float* __restrict__ Umat, int64_t u_layer_stride, const float* __restrict__ logP,
    int64_t logp_layer_stride, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t B,
    int32_t N, int32_t H, int32_t d_k, int32_t d_v, uint32_t* __restrict__ err) {
  __shared__ int pj[kMaxTree];
  __shared__ float wj[kMaxTree];

  const int unit = blockIdx.x;
  const int layer = blockIdx.y;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int a = accept[b];
  if (a == -1) return;
  const bool report_here = threadIdx.x == 0 && h == 0 && layer == 0;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (report_here) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (a < 0 || a >= T) {
    if (report_here) report(err, BOLE_ERR_BAD_ACCEPT);
    return;
  }
  const int s = slot[b];
  if (s < 0 || s >= n_slots) {
    if (report_here) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const float* lp = logP + layer * logp_layer_stride;
  const float* Ul = Umat + layer * u_layer_stride;
  const void* kl = DT == BOLE_BF16
                       ? (const void*)(reinterpret_cast<const uint16_t*>(kmat) + layer * k_layer_stride)
                       : (const void*)(reinterpret_cast<const float*>(kmat) + layer * k_layer_stride);
  float* S = state_pool + layer * state_layer_stride + ((int64_t)s * H + h) * d_v * d_k;

  const uint64_t tmask = T == 64 ? ~0ull : ((1ull << T) - 1ull);
  const uint64_t path = anc[off + a] & tmask;
  const int La = __popcll(path);
  const float lpa = lp[(int64_t)(off + a) * H + h];
  const float Pa = expf(lpa);
  if (threadIdx.x < kMaxTree && ((path >> threadIdx.x) & 1ull)) {
    const int t = threadIdx.x;
    const int p = __popcll(path & ((1ull << t) - 1ull));
    pj[p] = t;
    wj[p] = expf(lpa - lp[(int64_t)(off + t) * H + h]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = 8 * (lane >> 4);
  const int n_mt = d_v >> 4, n_nt = d_k >> 4;
  const int64_t krow = (int64_t)H * d_k;  // element stride between node rows of k
  for (int mt = w; mt < n_mt; mt += 4) {
    const int vrow = 16 * mt + (lane & 15);
    for (int ng = 0; ng < n_nt; ng += 8) {
      f32x4 acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kc = 0; kc < La; kc += 32) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = kc + kgrp + e;
          x[e] = p < La ? wj[p] * Ul[((int64_t)(off + pj[p]) * H + h) * d_v + vrow] : 0.0f;
        }
        bf16x8 a_hi, a_lo;
        split_bf16x8(x, a_hi, a_lo);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (ng + t < n_nt) {
            const int c = 16 * (ng + t) + (lane & 15);
            bf16x8 b_hi, b_lo;
            load_key8<DT>(kl, krow, pj, kc + kgrp, La, (int64_t)off * krow + (int64_t)h * d_k,
                          c, b_hi, b_lo);
            acc[t] = mfma_bf16(a_hi, b_hi, acc[t]);
            acc[t] = mfma_bf16(a_lo, b_hi, acc[t]);
            if (DT == BOLE_F32) acc[t] = mfma_bf16(a_hi, b_lo, acc[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (ng + t < n_nt) {
          const int c = 16 * (ng + t) + (lane & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vv = 16 * mt + 4 * (lane >> 4) + e;
            float* ps = S + (int64_t)vv * d_k + c;
            *ps = Pa * (*ps) + acc[t][e];
          }
        }
      }
    }
  }
}

}  // namespace bole

extern "C" int bole_commit_launch(int32_t L, float* state_pool, int64_t state_layer_stride,
                                  int32_t n_slots, const int32_t* slot, int32_t dtype,
                                  const void* k, int64_t k_layer_stride, const float* U,
                                  int64_t u_layer_stride, const float* logP,
                                  int64_t logp_layer_stride, const uint64_t* anc,
                                  const int32_t* tree_off, const int32_t* accept, int32_t B,
                                  int32_t N, int32_t H, int32_t d_k, int32_t d_v, uint32_t* err,
                                  hipStream_t s) {
  const dim3 grid(B * H, L), block(256);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_BF16>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, err);
  else
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_F32>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
