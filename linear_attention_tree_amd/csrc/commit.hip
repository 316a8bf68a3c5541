// Accepted-path state reconstruction (paper Eq. 10; review: one batched commit
// over all recurrent layers), in place on the state pool:
//
//   S[v][c] <- P_a S[v][c] + sum_{j in path(a)} (P_a/P_j) U_j[v] k_j[c]
//
// One single-wave workgroup per (layer, request, head, 64 value rows of the
// slot, 128 key columns): two 64x64 blocks A and B side by side.  Waves are
// independent: no LDS staging and no barrier.  Each wave issues block A's slot
// loads, derives the path from the ancestor mask and the gate sums held across
// its lanes, loads its operand fragments straight from global memory (a
// 16-lane group reads one contiguous row segment per load), and only then
// requests block B.  Loads complete in issue order, so block A is finished and
// stored while block B is still streaming in: the write of one block overlaps
// the read of the other.
//
// The path sum is a [d_k x L_a] x [L_a x d_v] product on
// v_mfma_f32_16x16x16_bf16 with the path position as K (steps of 16: a path is
// rarely longer, and each step's fragments are four loads per lane):
// A = k_j (bf16 exact; float32 keys split hi+lo), B = (P_a/P_j) U_j (float32,
// split hi+lo).  The accumulator of a 16x16 tile holds four consecutive key
// columns of one value row, which is one float4 of the slot: every slot
// element is read once and written once.  Each accumulator starts from P_a S
// (one float32 product) and the path steps add onto it, so the deferred
// commit inside bole_commit_tree_verify, which takes the same MFMA steps on the
// same operands, produces the same bits.
#include <type_traits>

#include "common.h"

namespace bole {

constexpr int kCommitBlk = 64;    // slot rows / columns per block
constexpr int kCommitTiles = 4;   // 16-wide tiles per block side
constexpr int kPathChunk = 16;    // path positions per MFMA K step
constexpr int kDppRowRor8 = 0x128;  // DPP control: rotate right by 8 within each 16-lane row

template <int DT>
struct CommitWave {
  using KRaw = std::conditional_t<DT == BOLE_BF16, uint16_t, uint32_t>;
  float* S;            // the (layer, slot, head) state, [d_v][d_k]
  const KRaw* kl;      // keys of the layer
  const float* Ul;     // U of the layer
  const int* pj;       // path position -> local node id
  const float* wj;     // path position -> P_a / P_j
  int64_t hk, hv;
  int off, H, d_k, d_v, La, v0, g4, l16;
  float Pa;

  // slot tiles of the block at key column c0; a tile past d_k or d_v (partial
  // block) reads tile (0, 0) of block A instead and is never stored, so every
  // load is unconditional and in bounds
  __device__ __forceinline__ void load_slot(int c0, int cA, f32x4 (&sv)[kCommitTiles][kCommitTiles]) const {
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt)
#pragma unroll
      for (int mt = 0; mt < kCommitTiles; ++mt) {
        const bool ok = tile_ok(c0, nt, mt);
        const int tv = ok ? v0 + 16 * nt : v0, tc = ok ? c0 + 16 * mt : cA;
        sv[nt][mt] = *reinterpret_cast<const f32x4*>(S + (tv + l16) * d_k + tc + 4 * g4);
      }
  }
  __device__ __forceinline__ bool tile_ok(int c0, int nt, int mt) const {
    return c0 + 16 * mt < d_k && v0 + 16 * nt < d_v;
  }

  // the lane's 4 path positions of the step starting at kc
  struct Step {
    int64_t rk[4], rv[4];
    float wt[4];
    bool live[4];
  };
  __device__ __forceinline__ Step step(int kc) const {
    Step st;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = kc + 4 * g4 + e;
      st.live[e] = p < La;
      const int node = st.live[e] ? pj[p] : 0;
      st.wt[e] = st.live[e] ? wj[p] : 0.0f;
      st.rk[e] = (int64_t)(off + node) * H * d_k + hk;
      st.rv[e] = (int64_t)(off + node) * H * d_v + hv;
    }
    return st;
  }
  // Fragment loads are unconditional (a dead position reads node 0, a column
  // past d_k reads c0, a row past d_v reads v0) and masked when converted.
  __device__ __forceinline__ void load_k(const Step& st, int c0, KRaw (&kraw)[kCommitTiles][4]) const {
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      const int c = c0 + 16 * mt + l16;
      const int cc = c < d_k ? c : c0;
#pragma unroll
      for (int e = 0; e < 4; ++e) kraw[mt][e] = kl[st.rk[e] + cc];
    }
  }
  __device__ __forceinline__ void load_u(const Step& st, float (&uraw)[kCommitTiles][4]) const {
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt) {
      const int v = v0 + 16 * nt + l16;
      const int vv = v < d_v ? v : v0;
#pragma unroll
      for (int e = 0; e < 4; ++e) uraw[nt][e] = Ul[st.rv[e] + vv];
    }
  }
  // B fragments: (P_a/P_j) U_j[v] for v = v0 + 16nt + l16, split hi+lo
  __device__ __forceinline__ void u_frags(const Step& st, const float (&uraw)[kCommitTiles][4],
                                          bf16x4 (&bh)[kCommitTiles], bf16x4 (&bl)[kCommitTiles]) const {
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt) {
      const bool vok = v0 + 16 * nt + l16 < d_v;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = __builtin_bit_cast(
            float, __builtin_bit_cast(uint32_t, st.wt[e] * uraw[nt][e]) & keep(st.live[e] && vok));
      split_bf16x4(x, bh[nt], bl[nt]);
    }
  }
  // D[c][v] += sum_p A[c][p] B[p][v], A = k_j[c] for c = c0 + 16mt + l16 (bf16
  // keys are exact)
  __device__ __forceinline__ void accumulate(const Step& st, int c0, const KRaw (&kraw)[kCommitTiles][4],
                                             const bf16x4 (&bh)[kCommitTiles], const bf16x4 (&bl)[kCommitTiles],
                                             f32x4 (&prod)[kCommitTiles][kCommitTiles]) const {
    bf16x4 ah[kCommitTiles], al[kCommitTiles];
#pragma unroll
    for (int mt = 0; mt < kCommitTiles; ++mt) {
      const bool cok = c0 + 16 * mt + l16 < d_k;
      if (DT == BOLE_BF16) {
        u16x4 raw;
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[e] = kraw[mt][e] & (uint16_t)keep(st.live[e] && cok);
        ah[mt] = __builtin_bit_cast(bf16x4, raw);
        al[mt] = bf16x4{};
      } else {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = __builtin_bit_cast(float, (uint32_t)kraw[mt][e] & keep(st.live[e] && cok));
        split_bf16x4(x, ah[mt], al[mt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt)
#pragma unroll
      for (int mt = 0; mt < kCommitTiles; ++mt) {
        prod[nt][mt] = mfma16_bf16(ah[mt], bh[nt], prod[nt][mt]);
        prod[nt][mt] = mfma16_bf16(ah[mt], bl[nt], prod[nt][mt]);
        if (DT == BOLE_F32) prod[nt][mt] = mfma16_bf16(al[mt], bh[nt], prod[nt][mt]);
      }
  }
  // the path product of the block at c0 over the steps from kc0 on
  __device__ __forceinline__ void product(int c0, int kc0, f32x4 (&prod)[kCommitTiles][kCommitTiles]) const {
    for (int kc = kc0; kc < La; kc += kPathChunk) {
      const Step st = step(kc);
      KRaw kraw[kCommitTiles][4];
      float uraw[kCommitTiles][4];
      load_k(st, c0, kraw);
      load_u(st, uraw);
      __builtin_amdgcn_sched_barrier(0);
      bf16x4 bh[kCommitTiles], bl[kCommitTiles];
      u_frags(st, uraw, bh, bl);
      accumulate(st, c0, kraw, bh, bl, prod);
    }
  }
  // Stores of whole 128-byte lines: tiles 2m and 2m+1 hold the two 64-byte
  // halves of rows 16nt + l16.  Exchanging tile 2m+1 between lanes l16 and
  // l16 ^ 8 (a row rotation by 8 within each 16-lane row) lets one store cover
  // rows 0..7 of the tile pair and the next rows 8..15, every row whole.  The
  // stores are written through the L2 (device scope): the slot lines were just
  // read into it, and left dirty there they would all be written back after
  // the last wave (measured 1.6 us slower at the target shape).
  __device__ __forceinline__ void init(const f32x4 (&sv)[kCommitTiles][kCommitTiles],
                                       f32x4 (&prod)[kCommitTiles][kCommitTiles]) const {
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt)
#pragma unroll
      for (int mt = 0; mt < kCommitTiles; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) prod[nt][mt][e] = Pa * sv[nt][mt][e];
  }
  __device__ __forceinline__ void store(int c0, const f32x4 (&prod)[kCommitTiles][kCommitTiles]) const {
    const bool lowh = l16 < 8;
#pragma unroll
    for (int nt = 0; nt < kCommitTiles; ++nt)
#pragma unroll
      for (int m = 0; m < kCommitTiles / 2; ++m) {
        const bool okX = tile_ok(c0, nt, 2 * m), okY = tile_ok(c0, nt, 2 * m + 1);
        if (!okX) continue;  // uniform; tile 2m+1 is past d_k too
        f32x4 oX, oY, oYr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          oX[e] = prod[nt][2 * m][e];
          // a scalar copy: the bit cast of a vector element itself would read element 0
          const float y = prod[nt][2 * m + 1][e];
          oY[e] = y;
          oYr[e] = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), kDppRowRor8, 0xf, 0xf,
                                                 false));
        }
        float* base = S + (v0 + 16 * nt) * d_k + c0 + 32 * m + 4 * g4;
        const int r1 = lowh ? l16 : l16 - 8, col1 = lowh ? 0 : 16;
        const int r2 = lowh ? l16 + 8 : l16, col2 = lowh ? 16 : 0;
        if (lowh || okY) store_sc1(base + r1 * d_k + col1, lowh ? oX : oYr);
        if (!lowh || okY) store_sc1(base + r2 * d_k + col2, lowh ? oYr : oX);
      }
  }
};

template <int DT>
__global__ __launch_bounds__(64) void commit_kernel(
    float* __restrict__ state_pool, int64_t state_layer_stride, int32_t n_slots,
    const int32_t* __restrict__ slot, const void* __restrict__ kmat, int64_t k_layer_stride,
    const float* __restrict__ Umat, int64_t u_layer_stride, const float* __restrict__ logP,
    int64_t logp_layer_stride, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t B,
    int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t n_bp, int32_t n_blk,
    uint32_t* __restrict__ err) {
  __shared__ int pj[kMaxTree];     // path position -> local node id (root first)
  __shared__ float wj[kMaxTree];   // path position -> P_a / P_j

  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = id / n_blk, blk = id - (id / n_blk) * n_blk;
  const int bv = blk / n_bp, bp = blk - (blk / n_bp) * n_bp;
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
  CommitWave<DT> cw;
  cw.g4 = lane >> 4;
  cw.l16 = lane & 15;
  cw.off = off;
  cw.H = H;
  cw.d_k = d_k;
  cw.d_v = d_v;
  cw.v0 = kCommitBlk * bv;
  cw.hk = (int64_t)h * d_k;
  cw.hv = (int64_t)h * d_v;
  cw.kl = reinterpret_cast<const typename CommitWave<DT>::KRaw*>(kmat) + layer * k_layer_stride;
  cw.Ul = Umat + layer * u_layer_stride;
  cw.S = state_pool + layer * state_layer_stride + ((int64_t)s * H + h) * d_v * d_k;
  cw.pj = pj;
  cw.wj = wj;
  const float* lp = logP + layer * logp_layer_stride;

  // gate sums of every tree node (one per lane; a lane past the tree reads node
  // T-1, unused) and the accepted node's mask
  const float lp_lane = lp[(int64_t)(off + min(lane, T - 1)) * H + h];
  const uint64_t tmask = T == 64 ? ~0ull : ((1ull << T) - 1ull);
  const uint64_t path = anc[off + a] & tmask;

  // Block A's slot tiles go out next, before the chain is waited on.  Block B
  // (key columns cA + 64 ..) exists when d_k > cA + 64.
  const int cA = 2 * kCommitBlk * bp, cB = cA + kCommitBlk;
  f32x4 svA[kCommitTiles][kCommitTiles], svB[kCommitTiles][kCommitTiles];
  cw.load_slot(cA, cA, svA);
  __builtin_amdgcn_sched_barrier(0);

  const float lpa = __shfl(lp_lane, a);
  cw.Pa = expf(lpa);
  cw.La = __popcll(path);
  if ((path >> lane) & 1ull) {
    const int p = __popcll(path & ((1ull << lane) - 1ull));
    pj[p] = lane;
    wj[p] = expf(lpa - lp_lane);
  }
  __syncthreads();  // a single wave: orders the LDS writes before the reads

  // The path products accumulate onto P_a S.
  f32x4 prod[kCommitTiles][kCommitTiles];
  const bool hasB = cB < d_k;  // uniform
  if (cw.La <= kPathChunk) {
    // one step: every fragment of both blocks is requested, then block B's
    // slot tiles, so block A's product and store wait for none of block B
    const typename CommitWave<DT>::Step st = cw.step(0);
    typename CommitWave<DT>::KRaw krA[kCommitTiles][4], krB[kCommitTiles][4];
    float uraw[kCommitTiles][4];
    cw.load_u(st, uraw);
    cw.load_k(st, cA, krA);
    cw.load_k(st, hasB ? cB : cA, krB);
    __builtin_amdgcn_sched_barrier(0);
    cw.load_slot(hasB ? cB : cA, cA, svB);
    __builtin_amdgcn_sched_barrier(0);
    bf16x4 bh[kCommitTiles], bl[kCommitTiles];
    cw.u_frags(st, uraw, bh, bl);
    cw.init(svA, prod);
    cw.accumulate(st, cA, krA, bh, bl, prod);
    cw.store(cA, prod);
    if (hasB) {
      cw.init(svB, prod);
      cw.accumulate(st, cB, krB, bh, bl, prod);
      cw.store(cB, prod);
    }
  } else {
    cw.init(svA, prod);
    cw.product(cA, 0, prod);
    cw.store(cA, prod);
    if (hasB) {
      cw.load_slot(cB, cA, svB);
      cw.init(svB, prod);
      cw.product(cB, 0, prod);
      cw.store(cB, prod);
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
  const int n_bp = (n_bc + 1) / 2;  // pairs of key-column blocks, one pair per wave
  const int n_bv = (d_v + bole::kCommitBlk - 1) / bole::kCommitBlk;
  const int n_blk = n_bp * n_bv;
  const dim3 grid(B * H * n_blk, L), block(64);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_BF16>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, n_bp,
                       n_blk, err);
  else
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_F32>, grid, block, 0, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, n_bp,
                       n_blk, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
