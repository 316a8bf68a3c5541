// G/C factor producer: one workgroup per (tree, head).
//
// G_ij = beta_i (P_i/P_j) k_i.k_j for j a strict ancestor of i (Lemma 2, Eq. 5)
// C_ij = (P_i/P_j) q_i.k_j        for j an ancestor of i or i   (Eq. 4)
// P_i/P_j = exp(logP_i - logP_j).  Rows and columns are indexed by level-order
// position (order[] of tree preparation), a parent-before-child indexing in
// which G is strictly lower triangular and C lower triangular.  The Gram
// products Q K^T and K K^T are dense 64x64xd_k contractions on bf16 MFMA with
// float32 accumulation (float32 q/k split into bf16 hi+lo); the ancestor mask,
// gate ratios and beta are applied in the epilogue.  Entries outside the mask
// are written as exact zeros.
//
// The tree's Q and K rows are staged once in LDS (level order, XOR-swizzled
// 16-byte chunks, every load in flight together).  Wave w owns rows
// [16w, 16w+16) of both products and sweeps the four 16-column blocks.
#include "common.h"

namespace bole {

constexpr int kGcThreads = 256;

template <int DT>
struct GcStage {
  static constexpr int KC = DT == BOLE_BF16 ? 128 : 64;  // d_k chunk per pass
  static constexpr int CHUNKS = KC / 8;                   // 16-byte chunks per row
  static constexpr int NMAT = DT == BOLE_BF16 ? 2 : 4;    // Q, K (hi) [+ lo]
};

template <int DT>
__device__ __forceinline__ int gc_swz(int row, int chunk) {
  return chunk ^ (row & (GcStage<DT>::CHUNKS - 1));
}

template <int DT>
__global__ __launch_bounds__(kGcThreads) void factor_gc_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ logP,
    const float* __restrict__ beta, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tree_off, int32_t B,
    int32_t N, int32_t H, int32_t d_k, float* __restrict__ G, float* __restrict__ C,
    uint32_t* __restrict__ err) {
  using SC = GcStage<DT>;
  __shared__ __align__(16) __bf16 stage[SC::NMAT * kMaxTree * SC::KC];
  __shared__ int rowNode[kMaxTree];
  __shared__ float rowLogP[kMaxTree];

  const int unit = xcd_remap(blockIdx.x, B * H);
  const int b = unit / H, h = unit - (unit / H) * H;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  float* Gt = G + (int64_t)unit * kMaxTree * kMaxTree;
  float* Ct = C + (int64_t)unit * kMaxTree * kMaxTree;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (threadIdx.x == 0 && h == 0) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (threadIdx.x < kMaxTree) rowNode[threadIdx.x] = lane < T ? clamp_node(order[off + lane], T) : 0;
  __syncthreads();

  // epilogue operands (small, issued before the staging loads are waited on)
  uint64_t ai[4];
  float lpi[4], bi[4], lpj[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * g4 + r;
    const int ni = rowNode[i];
    const bool iv = i < T;
    ai[r] = iv ? anc[off + ni] : 0ull;
    lpi[r] = iv ? logP[(int64_t)(off + ni) * H + h] : 0.0f;
    bi[r] = iv ? beta[(int64_t)(off + ni) * H + h] : 0.0f;
  }
  if (threadIdx.x < kMaxTree)
    rowLogP[threadIdx.x] = lane < T ? logP[(int64_t)(off + rowNode[lane]) * H + h] : 0.0f;

  f32x4 qk[4], kk[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    qk[nt] = zero_f32x4();
    kk[nt] = zero_f32x4();
  }
  const int nmt = (T + 15) >> 4;
  for (int kc0 = 0; kc0 < d_k; kc0 += SC::KC) {
    if (kc0 > 0) __syncthreads();
    // stage this chunk of Q and K rows (level order)
    constexpr int EPP = DT == BOLE_BF16 ? 8 : 4;
    constexpr int PIECES = SC::KC / EPP;
    constexpr int PER = 2 * kMaxTree * PIECES / kGcThreads;
    u16x8 buf[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int id = threadIdx.x + kGcThreads * it;
      const int mat = id / (kMaxTree * PIECES);
      const int rem = id - mat * (kMaxTree * PIECES);
      const int row = rem / PIECES, pc = rem - (rem / PIECES) * PIECES;
      const int kk2 = kc0 + EPP * pc;
      u16x8 val = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (row < T && kk2 < d_k) {
        const int64_t e = ((int64_t)(off + rowNode[row]) * H + h) * d_k + kk2;
        val = DT == BOLE_BF16
                  ? *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(mat ? k : q) + e)
                  : *reinterpret_cast<const u16x8*>(reinterpret_cast<const float*>(mat ? k : q) + e);
      }
      buf[it] = val;
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int id = threadIdx.x + kGcThreads * it;
      const int mat = id / (kMaxTree * PIECES);
      const int rem = id - mat * (kMaxTree * PIECES);
      const int row = rem / PIECES, pc = rem - (rem / PIECES) * PIECES;
      if (DT == BOLE_BF16) {
        *reinterpret_cast<u16x8*>(stage + (mat * kMaxTree + row) * SC::KC + 8 * gc_swz<DT>(row, pc)) =
            buf[it];
      } else {
        bf16x4 hi, lo;
        split_bf16x4(__builtin_bit_cast(f32x4, buf[it]), hi, lo);
        const int ch = gc_swz<DT>(row, pc >> 1), half = pc & 1;
        *reinterpret_cast<bf16x4*>(stage + (mat * kMaxTree + row) * SC::KC + 8 * ch + 4 * half) = hi;
        *reinterpret_cast<bf16x4*>(stage + ((2 + mat) * kMaxTree + row) * SC::KC + 8 * ch + 4 * half) =
            lo;
      }
    }
    __syncthreads();
    if (w < nmt) {
#pragma unroll
      for (int kk2 = 0; kk2 < SC::KC / 32; ++kk2) {
        if (kc0 + 32 * kk2 < d_k) {
          const int arow = 16 * w + l16;
          const int ao = arow * SC::KC + 8 * gc_swz<DT>(arow, 4 * kk2 + g4);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(stage + ao);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(stage + kMaxTree * SC::KC + ao);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            if (nt < nmt) {
              const int brow = 16 * nt + l16;
              const int bo = (kMaxTree + brow) * SC::KC + 8 * gc_swz<DT>(brow, 4 * kk2 + g4);
              const bf16x8 bk = *reinterpret_cast<const bf16x8*>(stage + bo);
              qk[nt] = mfma_bf16(aq, bk, qk[nt]);
              kk[nt] = mfma_bf16(ak, bk, kk[nt]);
              if (DT == BOLE_F32) {
                const int lo_off = 2 * kMaxTree * SC::KC;
                const bf16x8 aql = *reinterpret_cast<const bf16x8*>(stage + lo_off + ao);
                const bf16x8 akl =
                    *reinterpret_cast<const bf16x8*>(stage + lo_off + kMaxTree * SC::KC + ao);
                const bf16x8 bkl = *reinterpret_cast<const bf16x8*>(stage + lo_off + bo);
                qk[nt] = mfma_bf16(aq, bkl, qk[nt]);
                qk[nt] = mfma_bf16(aql, bk, qk[nt]);
                kk[nt] = mfma_bf16(ak, bkl, kk[nt]);
                kk[nt] = mfma_bf16(akl, bk, kk[nt]);
              }
            }
          }
        }
      }
    }
  }
  // epilogue: lane holds rows 16w + 4*(lane/16) + r, column 16nt + lane%16 (level
  // positions); the mask test is on the nodes those positions hold
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) lpj[nt] = rowLogP[16 * nt + l16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * g4 + r;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = 16 * nt + l16;
      const int nj = rowNode[j];
      float gv = 0.0f, cv = 0.0f;
      if (i < T && j < T && ((ai[r] >> nj) & 1ull)) {
        const float ratio = expf(lpi[r] - lpj[nt]);
        cv = ratio * qk[nt][r];
        if (j != i) gv = bi[r] * ratio * kk[nt][r];
      }
      Gt[i * kMaxTree + j] = gv;
      Ct[i * kMaxTree + j] = cv;
    }
  }
}

}  // namespace bole

extern "C" int bole_factor_gc_launch(int32_t dtype, const void* q, const void* k,
                                     const float* logP, const float* beta, const uint64_t* anc,
                                     const int32_t* order, const int32_t* tree_off, int32_t B,
                                     int32_t N, int32_t H, int32_t d_k, float* G, float* C,
                                     uint32_t* err, hipStream_t s) {
  const dim3 grid(B * H), block(bole::kGcThreads);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::factor_gc_kernel<BOLE_BF16>, grid, block, 0, s, q, k, logP, beta,
                       anc, order, tree_off, B, N, H, d_k, G, C, err);
  else
    hipLaunchKernelGGL(bole::factor_gc_kernel<BOLE_F32>, grid, block, 0, s, q, k, logP, beta,
                       anc, order, tree_off, B, N, H, d_k, G, C, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
