// Value-tiled closed-form verification (Bole, arXiv page section IV-B; the
// review's Eqs. 7 and 8).  One workgroup per (tree b, head h, value tile r) of
// kBV value columns; the tree is never split across workgroups.  Each of the
// eight waves owns 16 value columns and every node row, so after the operands
// are staged no wave ever waits for another.  At d_v = 128 a head is one
// workgroup and the whole forest fits on the chip in a single round.
//
// Rows are taken in level order (nodes sorted by depth, the order produced by
// tree preparation).  That is a parent-before-child indexing, so G is strictly
// lower triangular and C lower triangular (arXiv page, Theorem 1 discussion),
// and the rows of depth < m form a prefix that Z^(m) = (-G)^m R leaves at
// exactly zero (Lemma 3).  The kernel skips every 16x16 tile that structure
// makes zero.
//
//  Phase A  [Q;K] S_pre^(r) on v_mfma_f32_16x16x32_bf16: Q/K rows staged once
//           in LDS (level order), S_pre rows of the wave's columns loaded
//           straight into B fragments and split into bf16 hi+lo (float32 Q/K
//           are split too), float32 accumulation.
//           B0 = D_P QS and R = D_beta (V - D_P KS) in the accumulators.
//  Phase C  finite Neumann recursion of Eq. 8 on v_mfma_f32_16x16x32_bf16:
//           Z <- -G Z, U += Z for d_b steps.  With a permuted K order (see
//           load_tri_blocks) the B operand of a product is the lane's own
//           accumulator entries of two Z tiles, so Z and U never leave
//           registers.  G and Z are split into bf16 hi+lo, three products per
//           block (hi.hi + lo.hi + hi.lo), float32 accumulation.
//  Phase D  readout O = B0 + C U the same way; O (token dtype) and the compact
//           float32 U are written back to the nodes' rows.
#include "verify_tiles.h"

namespace bole {

// FUSED = false: G and C come from bole_factor_gc.  FUSED = true: the Gram
// products and their masked epilogue run here, from the Q/K rows already staged
// for the state contractions, with the same arithmetic as bole_factor_gc (d_k
// must fit one staged chunk).
template <int DT, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void verify_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ logP, const float* __restrict__ beta,
    const float* __restrict__ state_pool, int32_t n_slots, const int32_t* __restrict__ slot,
    const float* __restrict__ G, const float* __restrict__ C, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ order,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ tree_off,
    const int32_t* __restrict__ tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
    int32_t d_v, void* __restrict__ O, float* __restrict__ U, uint32_t* __restrict__ err) {
  using SC = StageCfg<DT>;
  __shared__ __align__(16) __bf16 stage[SC::NMAT * kMaxTree * SC::LROW];
  __shared__ __align__(16) __bf16 gcs[4 * kGcPlane];  // -G hi, -G lo, C hi, C lo
  __shared__ float rowP[kMaxTree], rowBeta[kMaxTree], rowLogP[kMaxTree];
  __shared__ uint64_t rowAnc[kMaxTree];
  __shared__ int rowNode[kMaxTree];
  static_assert(sizeof(stage) >= kWaves * 4 * 64 * sizeof(f32x4), "B0 parking space");

  const int NV = (d_v + kBV - 1) / kBV;
  const int lid = xcd_remap(blockIdx.x, B * H * NV);
  const int unit = lid / NV, r = lid - (lid / NV) * NV;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform
  const int g4 = lane >> 4, l16 = lane & 15;

  // G and C depend on the unit only: their loads go out first and are parked in
  // LDS once the operands below are in flight.  The fused variant clears the
  // planes instead (tiles above the diagonal are read and must be zero).
  constexpr int kGcPer = 2 * kMaxTree * kMaxTree / 4 / kThreads;  // float4 per thread
  f32x4 gcr[kGcPer];
  if (!FUSED) {
    const float* Gt = G + (int64_t)unit * kMaxTree * kMaxTree;
    const float* Ct = C + (int64_t)unit * kMaxTree * kMaxTree;
#pragma unroll
    for (int it = 0; it < kGcPer; ++it) {
      const int id = threadIdx.x + kThreads * it;       // float4 index over [G; C]
      const int mat = id >> 10, rem = id & 1023;
      gcr[it] = *reinterpret_cast<const f32x4*>((mat ? Ct : Gt) + 4 * rem);
    }
  } else {
#pragma unroll
    for (int it = 0; it < 4 * kGcPlane / 8 / kThreads; ++it)
      *reinterpret_cast<u16x8*>(gcs + 8 * (threadIdx.x + kThreads * it)) =
          u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // independent per-tree scalars, fetched together
  const int off = tree_off[b], end = tree_off[b + 1];
  const int td = tree_depth[b];
  const int s = slot[b];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (threadIdx.x == 0 && h == 0 && r == 0) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (td < 0) return;  // rejected by tree preparation
  if (s < 0 || s >= n_slots) {
    if (threadIdx.x == 0 && h == 0 && r == 0) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int d_b = min(td, T - 1);
  const int nmt = (T + 15) >> 4;

  // level-order rows: row p holds node order[p]
  const int node_l = lane < T ? clamp_node(order[off + lane], T) : 0;
  if (threadIdx.x < kMaxTree) rowNode[threadIdx.x] = node_l;
  __syncthreads();  // rowNode visible

  // everything below depends on the rows only: one round trip for all operands
  // depth of level-order row `lane` (nondecreasing in the row index)
  const int dep_row = lane < T ? depth[off + node_l] : 0x7fff;
  float lp_l = 0.0f, bt_l = 0.0f;
  uint64_t an_l = 0ull;
  if (threadIdx.x < kMaxTree && lane < T) {
    const int64_t tok = (int64_t)(off + node_l) * H + h;
    lp_l = logP[tok];
    bt_l = beta[tok];
    if (FUSED) an_l = anc[off + node_l];
  }

  // S_pre rows of this wave's 16 value columns: first chunk's B fragments
  const int vloc = 16 * w + l16;
  const int vcol = kBV * r + vloc;
  const bool vin = vcol < d_v;
  const float* Srow = state_pool + (((int64_t)s * H + h) * d_v + (vin ? vcol : 0)) * d_k;
  float sx[SC::KC / 32][8];
  auto load_s = [&](int kc0) {
#pragma unroll
    for (int kk = 0; kk < SC::KC / 32; ++kk) {
      const int kidx = kc0 + 32 * kk + 8 * g4;
      if (vin && kidx < d_k) {
        load_f32x8(Srow + kidx, sx[kk]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sx[kk][e] = 0.0f;
      }
    }
  };
  load_s(0);

  // this lane's V entries (accumulator layout), consumed after phase A
  float vv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 16 * mt + 4 * g4 + e;
      vv[mt][e] = (mt < nmt && p < T && vin)
                      ? load_scalar<DT>(v, ((int64_t)(off + rowNode[p]) * H + h) * d_v + vcol)
                      : 0.0f;
    }

  // park G (negated) and C in LDS, split once into bf16 hi/lo planes
#pragma unroll
  for (int it = 0; it < (FUSED ? 0 : kGcPer); ++it) {
    const int id = threadIdx.x + kThreads * it;
    const int mat = id >> 10, rem = id & 1023;
    const int row = rem >> 4, c4 = rem & 15;
    bf16x4 hi, lo;
    split_bf16x4(mat ? gcr[it] : -gcr[it], hi, lo);
    const int o = gc_pos(row, 4 * c4);
    *reinterpret_cast<bf16x4*>(gcs + (2 * mat) * kGcPlane + o) = hi;
    *reinterpret_cast<bf16x4*>(gcs + (2 * mat + 1) * kGcPlane + o) = lo;
  }
  if (threadIdx.x < kMaxTree) {
    rowP[threadIdx.x] = lane < T ? expf(lp_l) : 0.0f;
    rowBeta[threadIdx.x] = bt_l;
    rowLogP[threadIdx.x] = lp_l;
    rowAnc[threadIdx.x] = an_l;
  }

  // ---------------- Phase A: [Q;K] S_pre^(r) ----------------
  f32x4 qs[4], ks[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    qs[mt] = zero_f32x4();
    ks[mt] = zero_f32x4();
  }
  for (int kc0 = 0; kc0 < d_k; kc0 += SC::KC) {
    if (kc0 > 0) {
      __syncthreads();  // every wave is done with the previous chunk
      load_s(kc0);
    }
    stage_qk<DT>(stage, q, k, rowNode, T, off, H, h, d_k, kc0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SC::KC / 32; ++kk) {
      if (kc0 + 32 * kk < d_k) {
        bf16x8 b_hi, b_lo;
        split_bf16x8(sx[kk], b_hi, b_lo);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mt < nmt) {
            const int row = 16 * mt + l16;
            const int ro = row * SC::LROW + 8 * swz<DT>(row, 4 * kk + g4);
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(stage + ro);
            const bf16x8 ak = *reinterpret_cast<const bf16x8*>(stage + kMaxTree * SC::LROW + ro);
            qs[mt] = mfma_bf16(aq, b_hi, qs[mt]);
            qs[mt] = mfma_bf16(aq, b_lo, qs[mt]);
            ks[mt] = mfma_bf16(ak, b_hi, ks[mt]);
            ks[mt] = mfma_bf16(ak, b_lo, ks[mt]);
            if (DT == BOLE_F32) {
              const bf16x8 aql =
                  *reinterpret_cast<const bf16x8*>(stage + 2 * kMaxTree * SC::LROW + ro);
              const bf16x8 akl =
                  *reinterpret_cast<const bf16x8*>(stage + 3 * kMaxTree * SC::LROW + ro);
              qs[mt] = mfma_bf16(aql, b_hi, qs[mt]);
              ks[mt] = mfma_bf16(akl, b_hi, ks[mt]);
            }
          }
        }
      }
    }
  }
  if (FUSED) {
    // d_k fits one staged chunk (checked by the host): each Gram tile is
    // finished here.  Same operands and accumulation order as bole_factor_gc,
    // then its masked epilogue, written straight into the split planes.
#pragma unroll
    for (int jb = 0; jb < kJobsPerWave; ++jb) {
      const int job = w + kWaves * jb;
      if (job < 20) {
        const int I = kTileI[job >> 1], J = kTileJ[job >> 1];
        if (I < nmt) {
          const bool is_c = job & 1;
          const int arow = 16 * I + l16, brow = 16 * J + l16;
          const int amat = is_c ? 0 : 1;  // Q for C, K for G
          f32x4 acc = zero_f32x4();
#pragma unroll
          for (int kk = 0; kk < SC::KC / 32; ++kk) {
            if (32 * kk < d_k) {
              const int ao = (amat * kMaxTree + arow) * SC::LROW + 8 * swz<DT>(arow, 4 * kk + g4);
              const int bo = (kMaxTree + brow) * SC::LROW + 8 * swz<DT>(brow, 4 * kk + g4);
              const bf16x8 ah = *reinterpret_cast<const bf16x8*>(stage + ao);
              const bf16x8 bh = *reinterpret_cast<const bf16x8*>(stage + bo);
              acc = mfma_bf16(ah, bh, acc);
              if (DT == BOLE_F32) {
                const int lo_off = 2 * kMaxTree * SC::LROW;
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(stage + lo_off + ao);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(stage + lo_off + bo);
                acc = mfma_bf16(ah, bl, acc);
                acc = mfma_bf16(al, bh, acc);
              }
            }
          }
          const int j = 16 * J + l16;
          const int nj = rowNode[j];
          const float lpj = rowLogP[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g4 + e;
            float val = 0.0f;
            if (i < T && j < T && ((rowAnc[i] >> nj) & 1ull)) {
              const float ratio = expf(rowLogP[i] - lpj);
              if (is_c)
                val = ratio * acc[e];
              else if (j != i)
                val = -(rowBeta[i] * ratio * acc[e]);
            }
            const __bf16 hi = (__bf16)val;
            const int o = gc_pos(i, j) + (is_c ? 2 * kGcPlane : 0);
            gcs[o] = hi;
            gcs[o + kGcPlane] = (__bf16)(val - (float)hi);
          }
        }
      }
    }
  }

  // B0 = D_P QS, R = D_beta (V - D_P KS); rows beyond the tree are exact zeros.
  // B0 waits in the (now idle) staging area until the readout.
  f32x4 z[4], u[4];
  f32x4* b0s = reinterpret_cast<f32x4*>(stage) + w * 4 * 64 + lane;
  __syncthreads();  // all waves are done reading the staged Q/K; G/C planes complete

  // -G blocks of the Neumann recursion (A fragments, level order)
  bf16x8 gh[6], gl[6];
  load_tri_blocks(gcs, gcs + kGcPlane, nmt, lane, gh, gl);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 b0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 16 * mt + 4 * g4 + e;
      const float P = rowP[p], bt = rowBeta[p];
      b0[e] = P * qs[mt][e];
      z[mt][e] = bt * (vv[mt][e] - P * ks[mt][e]);
    }
    b0s[mt * 64] = b0;
    u[mt] = z[mt];
  }

  // ---------------- Phase C: Neumann recursion (Eq. 8) ----------------
  // Z <- (-G) Z, U += Z.  -G enters as hi + lo; Z as hi + lo for float32 token
  // inputs and as one rounded bf16 term for bf16 inputs (U accumulates in fp32).
  for (int m = 0; m < d_b; ++m) {
    // rows with depth >= m+1 start at tile I0; Z^(m) is zero before block J0
    const int I0 = __popcll(ballot64(dep_row < m + 1)) >> 4;
    const int J0 = __popcll(ballot64(dep_row < m)) >> 5;
    bf16x8 zh[2], zl[2];
#pragma unroll
    for (int J = 0; J < 2; ++J) {
      if (DT == BOLE_F32) {
        split_pair(z[2 * J], z[2 * J + 1], zh[J], zl[J]);
      } else {
        zh[J] = to_bf16x8(z[2 * J], z[2 * J + 1]);
        zl[J] = zero_bf16x8();
      }
    }
#pragma unroll
    for (int I = 3; I >= 0; --I) {
      f32x4 acc = zero_f32x4();
      if (I >= I0 && I < nmt) {
#pragma unroll
        for (int J = 0; J <= I / 2; ++J) {
          if (J >= J0) {
            const int idx = kBlk(I, J);
            acc = mfma_bf16(gh[idx], zh[J], acc);
            acc = mfma_bf16(gl[idx], zh[J], acc);
            if (DT == BOLE_F32) acc = mfma_bf16(gh[idx], zl[J], acc);
          }
        }
      }
      z[I] = acc;
      u[I] += acc;
    }
  }

  // ---------------- Phase D: readout O = B0 + C U ----------------
  bf16x8 ch[6], cl[6];
  load_tri_blocks(gcs + 2 * kGcPlane, gcs + 3 * kGcPlane, nmt, lane, ch, cl);
  bf16x8 uh[2], ul[2];
#pragma unroll
  for (int J = 0; J < 2; ++J) split_pair(u[2 * J], u[2 * J + 1], uh[J], ul[J]);
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    f32x4 acc = b0s[I * 64];
    if (I < nmt) {
#pragma unroll
      for (int J = 0; J <= I / 2; ++J) {
        const int idx = kBlk(I, J);
        acc = mfma_bf16(ch[idx], uh[J], acc);
        acc = mfma_bf16(cl[idx], uh[J], acc);
        acc = mfma_bf16(ch[idx], ul[J], acc);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 16 * I + 4 * g4 + e;
      if (I < nmt && p < T && vin) {
        const int64_t at = ((int64_t)(off + rowNode[p]) * H + h) * d_v + vcol;
        U[at] = u[I][e];
        store_scalar<DT>(O, at, acc[e]);
      }
    }
  }
}

}  // namespace bole

namespace {
template <bool FUSED>
int launch_verify(int32_t dtype, const void* q, const void* k, const void* v, const float* logP,
                  const float* beta, const float* state_pool, int32_t n_slots,
                  const int32_t* slot, const float* G, const float* C, const uint64_t* anc,
                  const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                  const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                  int32_t d_v, void* O, float* U, uint32_t* err, hipStream_t s) {
  const int NV = (d_v + bole::kBV - 1) / bole::kBV;
  const dim3 grid(B * H * NV), block(bole::kThreads);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL((bole::verify_kernel<BOLE_BF16, FUSED>), grid, block, 0, s, q, k, v, logP,
                       beta, state_pool, n_slots, slot, G, C, anc, order, depth, tree_off,
                       tree_depth, B, N, H, d_k, d_v, O, U, err);
  else
    hipLaunchKernelGGL((bole::verify_kernel<BOLE_F32, FUSED>), grid, block, 0, s, q, k, v, logP,
                       beta, state_pool, n_slots, slot, G, C, anc, order, depth, tree_off,
                       tree_depth, B, N, H, d_k, d_v, O, U, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
}  // namespace

extern "C" int bole_verify_launch(int32_t dtype, const void* q, const void* k, const void* v,
                                  const float* logP, const float* beta, const float* state_pool,
                                  int32_t n_slots, const int32_t* slot, const float* G,
                                  const float* C, const int32_t* order, const int32_t* depth,
                                  const int32_t* tree_off, const int32_t* tree_depth, int32_t B,
                                  int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O,
                                  float* U, uint32_t* err, hipStream_t s) {
  return launch_verify<false>(dtype, q, k, v, logP, beta, state_pool, n_slots, slot, G, C,
                              nullptr, order, depth, tree_off, tree_depth, B, N, H, d_k, d_v, O,
                              U, err, s);
}

extern "C" int bole_factor_verify_max_dk(int32_t dtype) {
  return dtype == BOLE_BF16 ? bole::StageCfg<BOLE_BF16>::KC : bole::StageCfg<BOLE_F32>::KC;
}

extern "C" int bole_factor_verify_launch(int32_t dtype, const void* q, const void* k,
                                         const void* v, const float* logP, const float* beta,
                                         const float* state_pool, int32_t n_slots,
                                         const int32_t* slot, const uint64_t* anc,
                                         const int32_t* order, const int32_t* depth,
                                         const int32_t* tree_off, const int32_t* tree_depth,
                                         int32_t B, int32_t N, int32_t H, int32_t d_k,
                                         int32_t d_v, void* O, float* U, uint32_t* err,
                                         hipStream_t s) {
  return launch_verify<true>(dtype, q, k, v, logP, beta, state_pool, n_slots, slot, nullptr,
                             nullptr, anc, order, depth, tree_off, tree_depth, B, N, H, d_k, d_v,
                             O, U, err, s);
}
