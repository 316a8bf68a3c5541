// G/C factor producer: one workgroup per (tree, head).
//
// G_ij = beta_i (P_i/P_j) k_i.k_j for j a strict ancestor of i (Lemma 2, Eq. 5)
// C_ij = (P_i/P_j) q_i.k_j        for j an ancestor of i or i   (Eq. 4)
// P_i/P_j = exp(logP_i - logP_j).  The Gram products Q K^T and K K^T are dense
// 64x64xd_k contractions on bf16 MFMA with float32 accumulation; the ancestor
// mask, gate ratios and beta are applied in the epilogue.  Entries outside the
// mask are written as exact zeros so downstream consumers may read any entry.
//
// Wave w owns rows [16w, 16w+16) of both tiles and sweeps all four 16-column
// blocks, so every K row fragment is loaded once per wave and reused.
#include "common.h"

namespace bole {

template <int DT>
__device__ __forceinline__ void load_row8(const void* base, int64_t elem, bool ok, bf16x8& hi,
                                          bf16x8& lo) {
  if (DT == BOLE_BF16) {
    hi = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(base) + elem) : zero_bf16x8();
  } else {
    float x[8];
    if (ok) {
      load_f32x8(reinterpret_cast<const float*>(base) + elem, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    split_bf16x8(x, hi, lo);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void factor_gc_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ logP,
    const float* __restrict__ beta, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
    float* __restrict__ G, float* __restrict__ C, uint32_t* __restrict__ err) {
  const int unit = xcd_remap(blockIdx.x, B * H);
  const int b = unit / H, h = unit - (unit / H) * H;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float* Gt = G + (int64_t)unit * kMaxTree * kMaxTree;
  float* Ct = C + (int64_t)unit * kMaxTree * kMaxTree;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (threadIdx.x == 0 && h == 0) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  const int row = 16 * w + (lane & 15);  // A-fragment row of this lane
  const int kgrp = 8 * (lane >> 4);      // K offset of this lane's 8 elements
  f32x4 qk[4], kk[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    qk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    kk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bool wave_live = 16 * w < T;
  if (wave_live) {
    for (int kc = 0; kc < d_k; kc += 32) {
      const int kidx = kc + kgrp;
      const bool kin = kidx < d_k;
      bf16x8 aq_hi, aq_lo, ak_hi, ak_lo;
      const bool rin = row < T && kin;
      const int64_t arow = ((int64_t)(off + row) * H + h) * d_k + kidx;
      load_row8<DT>(q, arow, rin, aq_hi, aq_lo);
      load_row8<DT>(k, arow, rin, ak_hi, ak_lo);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (16 * nt >= T) break;
        const int col = 16 * nt + (lane & 15);
        bf16x8 bk_hi, bk_lo;
        load_row8<DT>(k, ((int64_t)(off + col) * H + h) * d_k + kidx, col < T && kin, bk_hi,
                      bk_lo);
        qk[nt] = mfma_bf16(aq_hi, bk_hi, qk[nt]);
        kk[nt] = mfma_bf16(ak_hi, bk_hi, kk[nt]);
        if (DT == BOLE_F32) {
          qk[nt] = mfma_bf16(aq_hi, bk_lo, qk[nt]);
          qk[nt] = mfma_bf16(aq_lo, bk_hi, qk[nt]);
          kk[nt] = mfma_bf16(ak_hi, bk_lo, kk[nt]);
          kk[nt] = mfma_bf16(ak_lo, bk_hi, kk[nt]);
        }
      }
    }
  }
  // epilogue: lane holds rows 16w + 4*(lane/16) + r, column 16nt + lane%16
  const int col0 = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * (lane >> 4) + r;
    const bool iv = i < T;
    const uint64_t ai = iv ? anc[off + i] : 0ull;
    const float lpi = iv ? logP[(int64_t)(off + i) * H + h] : 0.0f;
    const float bi = iv ? beta[(int64_t)(off + i) * H + h] : 0.0f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = 16 * nt + col0;
      float gv = 0.0f, cv = 0.0f;
      if (iv && j < T && ((ai >> j) & 1ull)) {
        const float ratio = expf(lpi - logP[(int64_t)(off + j) * H + h]);
        cv = ratio * qk[nt][r];
        if (j != i) gv = bi * ratio * kk[nt][r];
      }
      Gt[i * kMaxTree + j] = gv;
      Ct[i * kMaxTree + j] = cv;
    }
  }
}

}  // namespace bole

extern "C" int bole_factor_gc_launch(int32_t dtype, const void* q, const void* k,
                                     const float* logP, const float* beta, const uint64_t* anc,
                                     const int32_t* tree_off, int32_t B, int32_t N, int32_t H,
                                     int32_t d_k, float* G, float* C, uint32_t* err,
                                     hipStream_t s) {
  const dim3 grid(B * H), block(256);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::factor_gc_kernel<BOLE_BF16>, grid, block, 0, s, q, k, logP, beta,
                       anc, tree_off, B, N, H, d_k, G, C, err);
  else
    hipLaunchKernelGGL(bole::factor_gc_kernel<BOLE_F32>, grid, block, 0, s, q, k, logP, beta,
                       anc, tree_off, B, N, H, d_k, G, C, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
