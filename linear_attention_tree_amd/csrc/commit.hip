// Accepted-path state reconstruction (paper Eq. 10; review: one batched commit
// over all recurrent layers), in place on the state pool:
//
//   S[v][c] <- P_a S[v][c] + sum_{j in path(a)} (P_a/P_j) U_j[v] k_j[c]
//
// One single-wave workgroup per (layer, request, head, 64x64 block of the
// slot).  Waves are independent: no LDS staging and no barrier.  Each wave
// issues its slot loads, derives the path from the ancestor mask and the gate
// sums held across its lanes, then loads its operand fragments straight from
// global memory (a 16-lane group reads one contiguous row segment per load).
//
// The path sum is a [d_k x L_a] x [L_a x d_v] product on
// v_mfma_f32_16x16x16_bf16 with the path position as K (steps of 16: a path is
// rarely longer, and each step's fragments are four loads per lane):
// A = k_j (bf16 exact; float32 keys split hi+lo), B = (P_a/P_j) U_j (float32,
// split hi+lo).  The accumulator of a 16x16 tile holds four consecutive key
// columns of one value row, which is one float4 of the slot: every slot
// element is read once and written once, as P_a S + the path product in
// float32.
#include <type_traits>

#include "common.h"

namespace bole {

constexpr int kCommitBlk = 64;    // slot rows / columns per wave
constexpr int kCommitTiles = 4;   // 16-wide tiles per block side
constexpr int kPathChunk = 16;    // path positions per MFMA K step

template <int DT>
__global__ __launch_bounds__(64) void commit_kernel(
    float* __restrict__ state_pool, int64_t state_layer_stride, int32_t n_slots,
    const int32_t* __restrict__ slot, const void* __restrict__ kmat, int64_t k_layer_stride,
    const float* __restrict__ Umat, int64_t u_layer_stride, const float* __restrict__ logP,
    int64_t logp_layer_stride, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t B,
    int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t n_bc, int32_t n_blk,
    uint32_t* __restrict__ err) {
  __shared__ int pj[kMaxTree];     // path position -> local node id (root first)
  __shared__ float wj[kMaxTree];   // path position -> P_a / P_j

  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = id / n_blk, blk = id - (id / n_blk) * n_blk;
  const int bv = blk / n_bc, bc = blk - (blk / n_bc) * n_bc;
  const int layer = blockIdx.y;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int a = accept[b];
  const int off = tree_off[b], end = tree_off[b + 1];
  const int s = slot[b];
  if (a == -1) return;
  // one reporter per request
  const bool reporter = threadIdx.x == 0 && h == 0 && blk == 0 && layer == 0;
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (reporter) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (a < 0 || a >= T) {
    if (reporter) report(err, BOLE_ERR_BAD_ACCEPT);
    return;
  }
  if (s < 0 || s >= n_slots) {
    if (reporter) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int lane = threadIdx.x;
  const int g4 = lane >> 4, l16 = lane & 15;
  const float* lp = logP + layer * logp_layer_stride;
  const float* Ul = Umat + layer * u_layer_stride;
  float* S = state_pool + layer * state_layer_stride + ((int64_t)s * H + h) * d_v * d_k;

  // gate sums of every tree node (one per lane; a lane past the tree reads node
  // T-1, unused) and the accepted node's mask
  const float lp_lane = lp[(int64_t)(off + min(lane, T - 1)) * H + h];
  const uint64_t tmask = T == 64 ? ~0ull : ((1ull << T) - 1ull);
  const uint64_t path = anc[off + a] & tmask;

  // The slot tiles go out next, before the chain is waited on (issued after
  // the chain, the commit was measured to finish later).  A tile past
  // d_k or d_v (partial block) reads tile (0, 0) instead and is never stored, so
  // every load is unconditional and in bounds.
  const int c0 = kCommitBlk * bc, v0 = kCommitBlk * bv;
  f32x4 prod[kCommitTiles][kCommitTiles], sv[kCommitTiles][kCommitTiles];
  bool tok[kCommitTiles][kCommitTiles];
#pragma unroll
  for (int nt = 0; nt < kCommitTiles; ++nt) {
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      prod[nt][mt] = zero_f32x4();
      tok[nt][mt] = c0 + 16 * mt < d_k && v0 + 16 * nt < d_v;
      const int tv = tok[nt][mt] ? 16 * nt : 0, tc = tok[nt][mt] ? 16 * mt : 0;
      sv[nt][mt] = *reinterpret_cast<const f32x4*>(S + (v0 + tv + l16) * d_k + c0 + tc + 4 * g4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const float lpa = __shfl(lp_lane, a);
  const float Pa = expf(lpa);
  const int La = __popcll(path);
  if ((path >> lane) & 1ull) {
    const int p = __popcll(path & ((1ull << lane) - 1ull));
    pj[p] = lane;
    wj[p] = expf(lpa - lp_lane);
  }
  __syncthreads();  // a single wave: orders the LDS writes before the reads

  // Tile (nt, mt) of this block covers value rows v0 + 16nt .. and key columns
  // c0 + 16mt ..; the lane's float4 is row 16nt + l16, columns 16mt + 4g4 .. +3.
  // The path products accumulate from zero; P_a S is added at the end.
  const int64_t hk = (int64_t)h * d_k, hv = (int64_t)h * d_v;
  for (int kc = 0; kc < La; kc += kPathChunk) {
    // the lane's 4 path positions of this step
    int64_t rk[4], rv[4];
    float wt[4];
    bool live[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = kc + 4 * g4 + e;
      live[e] = p < La;
      const int node = live[e] ? pj[p] : 0;
      wt[e] = live[e] ? wj[p] : 0.0f;
      rk[e] = (int64_t)(off + node) * H * d_k + hk;
      rv[e] = (int64_t)(off + node) * H * d_v + hv;
    }
    // Every fragment load of the step is issued before any value is used.
    // Loads are unconditional (a dead position reads node 0, a column past d_k
    // reads c0, a row past d_v reads v0) and masked afterwards.
    using KRaw = std::conditional_t<DT == BOLE_BF16, uint16_t, uint32_t>;
    KRaw kraw[kCommitTiles][4];
    float uraw[kCommitTiles][4];
    const KRaw* kl = reinterpret_cast<const KRaw*>(kmat) + layer * k_layer_stride;
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      const int c = c0 + 16 * mt + l16;
      const int cc = c < d_k ? c : c0;
#pragma unroll
      for (int e = 0; e < 4; ++e) kraw[mt][e] = kl[rk[e] + cc];
    }
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt) {
      const int v = v0 + 16 * nt + l16;
      const int vv = v < d_v ? v : v0;
#pragma unroll
      for (int e = 0; e < 4; ++e) uraw[nt][e] = Ul[rv[e] + vv];
    }
    __builtin_amdgcn_sched_barrier(0);
    // A fragments: k_j[c] for c = c0 + 16mt + l16 (bf16 keys are exact)
    bf16x4 ah[kCommitTiles], al[kCommitTiles];
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      const bool cok = c0 + 16 * mt + l16 < d_k;
      if (DT == BOLE_BF16) {
        u16x4 raw;
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[e] = kraw[mt][e] & (uint16_t)keep(live[e] && cok);
        ah[mt] = __builtin_bit_cast(bf16x4, raw);
        al[mt] = bf16x4{};
      } else {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = __builtin_bit_cast(float, (uint32_t)kraw[mt][e] & keep(live[e] && cok));
        split_bf16x4(x, ah[mt], al[mt]);
      }
    }
    // B fragments: (P_a/P_j) U_j[v] for v = v0 + 16nt + l16, split hi+lo
    bf16x4 bh[kCommitTiles], bl[kCommitTiles];
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt) {
      const bool vok = v0 + 16 * nt + l16 < d_v;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = __builtin_bit_cast(
            float, __builtin_bit_cast(uint32_t, wt[e] * uraw[nt][e]) & keep(live[e] && vok));
      split_bf16x4(x, bh[nt], bl[nt]);
    }
    // D[c][v] += sum_p A[c][p] B[p][v]
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt) {
#pragma unroll
      for (int mt = 0; mt < kCommitTiles; ++mt) {
        prod[nt][mt] = mfma16_bf16(ah[mt], bh[nt], prod[nt][mt]);
        prod[nt][mt] = mfma16_bf16(ah[mt], bl[nt], prod[nt][mt]);
        if (DT == BOLE_F32) prod[nt][mt] = mfma16_bf16(al[mt], bh[nt], prod[nt][mt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < kCommitTiles; ++nt) {
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      if (tok[nt][mt]) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = Pa * sv[nt][mt][e] + prod[nt][mt][e];
        *reinterpret_cast<f32x4*>(S + (v0 + 16 * nt + l16) * d_k + c0 + 16 * mt + 4 * g4) = o;
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
  const int n_bc = (d_k + bole::kCommitBlk - 1) / bole::kCommitBlk;
  const int n_bv = (d_v + bole::kCommitBlk - 1) / bole::kCommitBlk;
  const int n_blk = n_bc * n_bv;
  const dim3 grid(B * H * n_blk, L), block(64);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_BF16>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, n_bc,
                       n_blk, err);
  else
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_F32>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, n_bc,
                       n_blk, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
