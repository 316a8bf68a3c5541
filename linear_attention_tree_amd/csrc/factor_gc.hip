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
//
// The INV variant (bole_factor_inverse) goes on to an explicit inverse, one of
// the exact solves the closed form allows: with N = -G, nilpotent of index at
// most d + 1 (Lemma 3), W = (I + G)^-1 = sum_{m<=d} N^m is formed by repeated
// squaring, W = prod_k (I + N^(2^k)) for 2^k <= d, and then M = C W.  It writes
// W and M in place of G and C, so a verify needs U = W R and O = B0 + M R only.
#include <algorithm>

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

// Row stride (floats) of a 64x64 float32 matrix held in LDS by the INV variant.
constexpr int kLd = kMaxTree + 4;

// acc[nt] (nt <= w) = sum_{kt = nt..w} X(w, kt) Y(kt, nt) over 16x16 tiles of
// two lower-triangular 64x64 matrices, on v_mfma_f32_16x16x16_bf16 with each
// operand split bf16 hi + lo (three products, float32 accumulation).  xfrag(kt)
// returns X's tile (w, kt) in the A layout (row l16, columns 4g .. 4g+3); Y is
// read from LDS in the B layout (rows 4g .. 4g+3, column l16).  The result is in
// the accumulator layout (rows 4g .. 4g+3, column l16).  Tiles above the
// diagonal are left at zero.
template <typename XFrag>
__device__ __forceinline__ void tri_mm(XFrag xfrag, const float* Y, int w, int lane, f32x4* acc) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = zero_f32x4();
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    if (kt <= w) {
      bf16x4 xh, xl;
      split_bf16x4(xfrag(kt), xh, xl);
#pragma unroll
      for (int nt = 0; nt <= kt; ++nt) {
        f32x4 yb;
#pragma unroll
        for (int e = 0; e < 4; ++e) yb[e] = Y[(16 * kt + 4 * g4 + e) * kLd + 16 * nt + l16];
        bf16x4 yh, yl;
        split_bf16x4(yb, yh, yl);
        acc[nt] = mfma16_bf16(xh, yh, acc[nt]);
        acc[nt] = mfma16_bf16(xl, yh, acc[nt]);
        acc[nt] = mfma16_bf16(xh, yl, acc[nt]);
      }
    }
  }
}

template <int DT, bool INV = false>
__global__ __launch_bounds__(kGcThreads) void factor_gc_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ logP,
    const float* __restrict__ beta, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tree_off, int32_t B,
    int32_t N, int32_t H, int32_t d_k, float* __restrict__ G, float* __restrict__ C,
    uint32_t* __restrict__ err) {
  using SC = GcStage<DT>;
  // the INV variant reuses the staging space for three float32 matrices once
  // the Gram products are done
  constexpr int kStageBytes = SC::NMAT * kMaxTree * SC::KC * 2;
  constexpr int kMatFloats = kMaxTree * kLd;
  constexpr int kSmem = INV ? std::max(kStageBytes, 3 * kMatFloats * 4) : kStageBytes;
  __shared__ __align__(16) char smem[kSmem];
  __bf16* stage = reinterpret_cast<__bf16*>(smem);
  __shared__ int wmax[4];
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
  f32x4 gv[4], cv[4];  // row i, columns 16nt + 4g .. +3: the A layout of tile (w, nt)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int j0 = 16 * nt + 4 * g4;
    const uint32_t m4 = (uint32_t)(apos >> j0) & 15u;
    const uint32_t d = (uint32_t)(i - j0);
    const uint32_t m4g = m4 & ~(d < 4u ? 1u << d : 0u);  // G has no diagonal
    const f32x4 e2j = *reinterpret_cast<const f32x4*>(rowE2 + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c1 = gate_ratio(e2i, e2j[e]) * qk[nt][e];
      const float g1 = bi * gate_ratio(e2i, e2j[e]) * kk[nt][e];
      cv[nt][e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c1) & keep((m4 >> e) & 1u));
      gv[nt][e] =
          __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, g1) & keep((m4g >> e) & 1u));
    }
    if (!INV) {
      *reinterpret_cast<f32x4*>(Gt + i * kMaxTree + j0) = gv[nt];
      *reinterpret_cast<f32x4*>(Ct + i * kMaxTree + j0) = cv[nt];
    }
  }
  if (!INV) return;

  // ---------------- W = (I + G)^-1 by repeated squaring, M = C W ----------------
  // The tree depth d is the deepest row's strict-ancestor count.
  int dep = __popcll(apos) - 1;  // -1 past the tree
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dep = max(dep, __shfl_xor(dep, o));
  if (lane == 0) wmax[w] = dep;
  __syncthreads();  // staged rows no longer read (their space is reused); wmax visible
  const int dtree = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  float* Pcur = reinterpret_cast<float*>(smem);
  float* Pnext = Pcur + kMatFloats;
  float* Wm = Pcur + 2 * kMatFloats;
  // N = -G and W = I + N, the wave's own rows (A layout)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = -gv[nt][e] + (16 * nt + 4 * g4 + e == i ? 1.0f : 0.0f);
    *reinterpret_cast<f32x4*>(Pcur + i * kLd + 16 * nt + 4 * g4) = -gv[nt];
    *reinterpret_cast<f32x4*>(Wm + i * kLd + 16 * nt + 4 * g4) = wv;
  }
  __syncthreads();  // N complete
  auto lds_rows = [&](const float* X) {
    return [=](int kt) { return *reinterpret_cast<const f32x4*>(X + i * kLd + 16 * kt + 4 * g4); };
  };
  f32x4 acc[4];
  // W holds N^0 .. N^cover; each round squares P = N^(2^s) and multiplies W by
  // (I + P), doubling the cover.  One barrier per round: the next round's
  // squaring writes the buffer this round's squaring read.
  for (int cover = 1; cover < dtree; cover = 2 * cover + 1) {
    tri_mm(lds_rows(Pcur), Pcur, w, lane, acc);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Pnext[(16 * w + 4 * g4 + e) * kLd + 16 * nt + l16] = acc[nt][e];
    __syncthreads();  // P^2 complete
    // W <- W + W P^2: only the wave's own rows of W are read and written
    tri_mm(lds_rows(Wm), Pnext, w, lane, acc);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* at = Wm + (16 * w + 4 * g4 + e) * kLd + 16 * nt + l16;
        if (nt <= w) *at += acc[nt][e];
      }
    float* t = Pcur;
    Pcur = Pnext;
    Pnext = t;
  }
  __syncthreads();  // W complete
  // M = C W, with C's tiles straight from the epilogue registers
  tri_mm([&](int kt) { return cv[kt]; }, Wm, w, lane, acc);
  // W leaves by rows (A layout), M in the accumulator layout; rows past the
  // tree and tiles above the diagonal are written as zeros
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const f32x4 wv = *reinterpret_cast<const f32x4*>(Wm + i * kLd + 16 * nt + 4 * g4);
    *reinterpret_cast<f32x4*>(Gt + i * kMaxTree + 16 * nt + 4 * g4) =
        iv && nt <= w ? wv : zero_f32x4();
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Ct[(16 * w + 4 * g4 + e) * kMaxTree + 16 * nt + l16] = nt <= w ? acc[nt][e] : 0.0f;
  }
}

}  // namespace bole

extern "C" int bole_factor_inverse_launch(int32_t dtype, const void* q, const void* k,
                                          const float* logP, const float* beta,
                                          const uint64_t* anc, const int32_t* order,
                                          const int32_t* tree_off, int32_t B, int32_t N,
                                          int32_t H, int32_t d_k, float* W, float* M,
                                          uint32_t* err, hipStream_t s) {
  const dim3 grid(B * H), block(bole::kGcThreads);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL((bole::factor_gc_kernel<BOLE_BF16, true>), grid, block, 0, s, q, k, logP,
                       beta, anc, order, tree_off, B, N, H, d_k, W, M, err);
  else
    hipLaunchKernelGGL((bole::factor_gc_kernel<BOLE_F32, true>), grid, block, 0, s, q, k, logP,
                       beta, anc, order, tree_off, B, N, H, d_k, W, M, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}

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
