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
  __shared__ int posOf[kMaxTree];  // local node id -> level position
  __shared__ __align__(16) float rowE2[kMaxTree];

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
  const int ord = order[off + min(lane, T - 1)];
  const int node_l = lane < T ? clamp_node(ord, T) : 0;
  if (threadIdx.x < kMaxTree) {
    rowNode[threadIdx.x] = node_l;
    if (lane < T) posOf[node_l] = lane;
  }
  __syncthreads();

  // The products are taken transposed (key rows of column tile nt as the M
  // operand), so a lane holds row i = 16w + l16 at the four consecutive columns
  // 16nt + 4g .. +3: one float4 store per tile and matrix.  Operand order,
  // accumulation order and epilogue arithmetic are those of the fused factor +
  // verify kernel, which makes the two paths' G and C bit-identical.
  const int i = 16 * w + l16;
  const bool iv = i < T;
  const int ni = rowNode[i];
  // epilogue operands of the lane's row: unconditional loads (ni is a valid
  // node), issued before the staging loads are waited on
  const uint64_t an_raw = anc[off + ni];
  const float lp_raw = logP[(int64_t)(off + ni) * H + h];
  const float bt_raw = beta[(int64_t)(off + ni) * H + h];
  const float e2i = lp_raw * kLog2e;
  const float bi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, bt_raw) & keep(iv));
  if (g4 == 0)
    rowE2[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e2i) & keep(iv));
  // the row's ancestor mask moved from node ids to level positions, where four
  // consecutive columns are four consecutive bits
  uint64_t apos = 0ull;
  {
    uint64_t m = an_raw & (T == 64 ? ~0ull : ((1ull << T) - 1ull));
    while (m) {
      apos |= 1ull << posOf[__builtin_ctzll(m)];
      m &= m - 1ull;
    }
    apos &= 0ull - (uint64_t)iv;
  }

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
      // unconditional load (row and column clamped into the tree), zeroed after
      const bool in = row < T && kk2 < d_k;
      const int64_t e =
          ((int64_t)(off + rowNode[min(row, T - 1)]) * H + h) * d_k + (kk2 < d_k ? kk2 : 0);
      const u16x8 val =
          DT == BOLE_BF16
              ? *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(mat ? k : q) + e)
              : *reinterpret_cast<const u16x8*>(reinterpret_cast<const float*>(mat ? k : q) + e);
      const u16x8 zero = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      buf[it] = in ? val : zero;
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
          const int ao = i * SC::KC + 8 * gc_swz<DT>(i, 4 * kk2 + g4);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(stage + ao);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(stage + kMaxTree * SC::KC + ao);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            if (nt < nmt && nt <= w) {
              const int brow = 16 * nt + l16;
              const int bo = (kMaxTree + brow) * SC::KC + 8 * gc_swz<DT>(brow, 4 * kk2 + g4);
              const bf16x8 bk = *reinterpret_cast<const bf16x8*>(stage + bo);
              qk[nt] = mfma_bf16(bk, aq, qk[nt]);
              kk[nt] = mfma_bf16(bk, ak, kk[nt]);
              if (DT == BOLE_F32) {
                const int lo_off = 2 * kMaxTree * SC::KC;
                const bf16x8 aql = *reinterpret_cast<const bf16x8*>(stage + lo_off + ao);
                const bf16x8 akl =
                    *reinterpret_cast<const bf16x8*>(stage + lo_off + kMaxTree * SC::KC + ao);
                const bf16x8 bkl = *reinterpret_cast<const bf16x8*>(stage + lo_off + bo);
                qk[nt] = mfma_bf16(bkl, aq, qk[nt]);
                qk[nt] = mfma_bf16(bk, aql, qk[nt]);
                kk[nt] = mfma_bf16(bkl, ak, kk[nt]);
                kk[nt] = mfma_bf16(bk, akl, kk[nt]);
              }
            }
          }
        }
      }
    }
  }
  // epilogue, branch-free: every entry is computed and the mask clears the ones
  // outside it (an overflowing ratio there is cleared too)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int j0 = 16 * nt + 4 * g4;
    const uint32_t m4 = (uint32_t)(apos >> j0) & 15u;
    const uint32_t d = (uint32_t)(i - j0);
    const uint32_t m4g = m4 & ~(d < 4u ? 1u << d : 0u);  // G has no diagonal
    const f32x4 e2j = *reinterpret_cast<const f32x4*>(rowE2 + j0);
    f32x4 gv, cv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c1 = gate_ratio(e2i, e2j[e]) * qk[nt][e];
      const float g1 = bi * gate_ratio(e2i, e2j[e]) * kk[nt][e];
      cv[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c1) & keep((m4 >> e) & 1u));
      gv[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, g1) & keep((m4g >> e) & 1u));
    }
    *reinterpret_cast<f32x4*>(Gt + i * kMaxTree + j0) = gv;
    *reinterpret_cast<f32x4*>(Ct + i * kMaxTree + j0) = cv;
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
