// Accepted-path state reconstruction (paper Eq. 10; review: one batched commit
// over all recurrent layers), in place on the state pool:
//
//   S[v][c] <- P_a S[v][c] + sum_{j in path(a)} (P_a/P_j) U_j[v] k_j[c]
//
// One workgroup per (layer, request, head).  The path sum is a
// [d_k x L_a] x [L_a x d_v] product on v_mfma_f32_16x16x32_bf16 with the path
// position as K (chunks of 32): A = k_j (bf16 exact; float32 keys split hi+lo),
// B = (P_a/P_j) U_j (float32, split hi+lo).  The path rows are staged once in
// LDS, transposed so every fragment is one 16-byte read.  The accumulator of a
// 16x16 tile holds four consecutive key columns of one value row, which is one
// float4 of the slot: each slot element is read once (prefetched before the
// products) and written once, with the P_a S term applied in float32.
#include "common.h"

namespace bole {

constexpr int kCommitThreads = 256;
constexpr int kPathChunk = 32;             // path positions per K chunk
constexpr int kPRow = kPathChunk + 8;      // bf16 per transposed LDS row (16 B pad)

template <int DT>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    float* __restrict__ state_pool, int64_t state_layer_stride, int32_t n_slots,
    const int32_t* __restrict__ slot, const void* __restrict__ kmat, int64_t k_layer_stride,
    const float* __restrict__ Umat, int64_t u_layer_stride, const float* __restrict__ logP,
    int64_t logp_layer_stride, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t B,
    int32_t N, int32_t H, int32_t d_k, int32_t d_v, uint32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int pj[kMaxTree];
  __shared__ float wj[kMaxTree];

  const int unit = blockIdx.x;
  const int layer = blockIdx.y;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int a = accept[b];
  const int off = tree_off[b], end = tree_off[b + 1];
  const int s = slot[b];
  if (a == -1) return;
  const bool report_here = threadIdx.x == 0 && h == 0 && layer == 0;
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (report_here) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (a < 0 || a >= T) {
    if (report_here) report(err, BOLE_ERR_BAD_ACCEPT);
    return;
  }
  if (s < 0 || s >= n_slots) {
    if (report_here) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const float* lp = logP + layer * logp_layer_stride;
  const float* Ul = Umat + layer * u_layer_stride;
  float* S = state_pool + layer * state_layer_stride + ((int64_t)s * H + h) * d_v * d_k;

  // transposed path planes: Kt[c][p] (hi[, lo]) and Wt[v][p] (hi, lo), bf16
  __bf16* Kt_hi = reinterpret_cast<__bf16*>(smem);
  __bf16* Kt_lo = Kt_hi + d_k * kPRow;
  __bf16* Wt_hi = Kt_lo + (DT == BOLE_F32 ? d_k * kPRow : 0);
  __bf16* Wt_lo = Wt_hi + d_v * kPRow;

  // Wave 0 walks the dependent chain (ancestor mask -> gate ratios -> path
  // rows) while the other waves already stream their slot tiles; a wave's
  // loads complete in issue order, so the chain must not queue behind them.
  __shared__ int La_s;
  __shared__ float Pa_s;
  // Path rows of one 32-position chunk -> transposed bf16 planes, wave 0 only.
  // Every load of a batch is issued before the batch is converted and stored,
  // so a chunk costs one or two memory round trips.
  auto stage_chunk = [&](int kc, int La) {
    constexpr int EPK = DT == BOLE_BF16 ? 8 : 4;  // key elements per 16-byte piece
    const int kp = d_k / EPK, up = d_v >> 2;       // pieces per key row / U row
    const int per_row = kp + up;
    const int total = kPathChunk * per_row;
    constexpr int kBatch = 16;
    for (int base = 0; base < total; base += 64 * kBatch) {
      u16x8 buf[kBatch];
#pragma unroll
      for (int it = 0; it < kBatch; ++it) {
        const int id = base + lane + 64 * it;
        const int p = id / per_row, q = id - (id / per_row) * per_row;
        const int pg = kc + p;
        const bool live = id < total && pg < La;
        const int node = live ? pj[pg] : 0;
        const int64_t row = (int64_t)(off + node) * H + h;
        buf[it] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (live) {
          if (q < kp) {
            buf[it] = DT == BOLE_BF16
                          ? *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(kmat) +
                                                            layer * k_layer_stride + row * d_k +
                                                            EPK * q)
                          : *reinterpret_cast<const u16x8*>(reinterpret_cast<const float*>(kmat) +
                                                            layer * k_layer_stride + row * d_k +
                                                            EPK * q);
          } else {
            buf[it] = *reinterpret_cast<const u16x8*>(Ul + row * d_v + 4 * (q - kp));
          }
        }
      }
#pragma unroll
      for (int it = 0; it < kBatch; ++it) {
        const int id = base + lane + 64 * it;
        if (id < total) {
          const int p = id / per_row, q = id - (id / per_row) * per_row;
          const int pg = kc + p;
          if (q < kp) {
            if (DT == BOLE_BF16) {
              const bf16x8 kv = __builtin_bit_cast(bf16x8, buf[it]);  // exact bf16 keys
#pragma unroll
              for (int e = 0; e < 8; ++e) Kt_hi[(EPK * q + e) * kPRow + p] = kv[e];
            } else {
              bf16x4 hi, lo;
              split_bf16x4(__builtin_bit_cast(f32x4, buf[it]), hi, lo);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                Kt_hi[(EPK * q + e) * kPRow + p] = hi[e];
                Kt_lo[(EPK * q + e) * kPRow + p] = lo[e];
              }
            }
          } else {
            const int v0 = 4 * (q - kp);
            const float wgt = pg < La ? wj[pg] : 0.0f;
            bf16x4 hi, lo;
            split_bf16x4(__builtin_bit_cast(f32x4, buf[it]) * wgt, hi, lo);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              Wt_hi[(v0 + e) * kPRow + p] = hi[e];
              Wt_lo[(v0 + e) * kPRow + p] = lo[e];
            }
          }
        }
      }
    }
  };
  if (w == 0) {
    const uint64_t tmask = T == 64 ? ~0ull : ((1ull << T) - 1ull);
    const uint64_t path = anc[off + a] & tmask;
    const float lpa = lp[(int64_t)(off + a) * H + h];
    if ((path >> lane) & 1ull) {
      const int p = __popcll(path & ((1ull << lane) - 1ull));
      pj[p] = lane;
      wj[p] = expf(lpa - lp[(int64_t)(off + lane) * H + h]);
    }
    if (lane == 0) {
      La_s = __popcll(path);
      Pa_s = expf(lpa);
    }
    // the wave's own LDS writes are visible to it in program order
    stage_chunk(0, __popcll(path));
  }

  // output tiles: value tile nt (16 slot rows) x key tile mt (16 columns), tile
  // id = nt * n_kt + mt; wave w owns ids w, w + 4, ... in groups of kGroup
  constexpr int kGroup = 16;
  const int n_vt = d_v >> 4, n_kt = d_k >> 4, n_tiles = n_vt * n_kt;
  const int per_wave = (n_tiles + 3) >> 2;
  const int n_groups = (per_wave + kGroup - 1) / kGroup;  // same for every wave
  int La = 0;
  float Pa = 0.0f;
  for (int grp = 0; grp < n_groups; ++grp) {
    f32x4 sv[kGroup], acc[kGroup];
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      const int tile = w + 4 * (grp * kGroup + t);
      acc[t] = zero_f32x4();
      sv[t] = zero_f32x4();
      if (tile < n_tiles) {
        const int nt = tile / n_kt, mt = tile - (tile / n_kt) * n_kt;
        sv[t] = *reinterpret_cast<const f32x4*>(S + (int64_t)(16 * nt + l16) * d_k + 16 * mt +
                                                 4 * g4);
      }
    }
    if (grp == 0) {
      __syncthreads();  // path planes of chunk 0, La, Pa ready
      La = La_s;
      Pa = Pa_s;
    }
    const int n_chunks = (La + kPathChunk - 1) / kPathChunk;
    for (int ch = 0; ch < n_chunks; ++ch) {
      // a chunk other than the one left in LDS must be (re)staged
      if (ch > 0 || (grp > 0 && n_chunks > 1)) {
        __syncthreads();  // previous chunk fully consumed
        if (w == 0) stage_chunk(ch * kPathChunk, La);
        __syncthreads();
      }
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        const int tile = w + 4 * (grp * kGroup + t);
        if (tile < n_tiles) {
          const int nt = tile / n_kt, mt = tile - (tile / n_kt) * n_kt;
          const bf16x8 ah =
              *reinterpret_cast<const bf16x8*>(Kt_hi + (16 * mt + l16) * kPRow + 8 * g4);
          const bf16x8 bh =
              *reinterpret_cast<const bf16x8*>(Wt_hi + (16 * nt + l16) * kPRow + 8 * g4);
          const bf16x8 bl =
              *reinterpret_cast<const bf16x8*>(Wt_lo + (16 * nt + l16) * kPRow + 8 * g4);
          acc[t] = mfma_bf16(ah, bh, acc[t]);
          acc[t] = mfma_bf16(ah, bl, acc[t]);
          if (DT == BOLE_F32) {
            const bf16x8 al =
                *reinterpret_cast<const bf16x8*>(Kt_lo + (16 * mt + l16) * kPRow + 8 * g4);
            acc[t] = mfma_bf16(al, bh, acc[t]);
          }
        }
      }
    }
    // D[c][v] of tile (mt, nt): lane holds c = 16mt + 4*g4 + e, v = 16nt + l16
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      const int tile = w + 4 * (grp * kGroup + t);
      if (tile < n_tiles) {
        const int nt = tile / n_kt, mt = tile - (tile / n_kt) * n_kt;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = Pa * sv[t][e] + acc[t][e];
        *reinterpret_cast<f32x4*>(S + (int64_t)(16 * nt + l16) * d_k + 16 * mt + 4 * g4) = o;
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
  const dim3 grid(B * H, L), block(bole::kCommitThreads);
  const size_t planes = (dtype == BOLE_F32 ? 2 : 1) * (size_t)d_k + 2 * (size_t)d_v;
  const size_t shm = planes * bole::kPRow * sizeof(uint16_t);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_BF16>, grid, block, shm, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, err);
  else
    hipLaunchKernelGGL(bole::commit_kernel<BOLE_F32>, grid, block, shm, s, state_pool,
                       state_layer_stride, n_slots, slot, k, k_layer_stride, U, u_layer_stride,
                       logP, logp_layer_stride, anc, tree_off, accept, B, N, H, d_k, d_v, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
