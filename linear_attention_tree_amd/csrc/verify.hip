// Value-tiled closed-form verification (Bole, arXiv page section IV-B; the
// review's Eqs. 7 and 8).  One workgroup per (tree b, head h, value tile r),
// tiles of kBV value columns; the tree is never split across workgroups.
//
//  Phase A  state contractions on MFMA.  Wave w owns 16 value columns of the
//           tile and all node rows: QS and KS = [Q;K] S_pre^(r) with the fp32
//           slot rows split into bf16 hi+lo parts (fp32 q/k are split too).
//           B0 = D_P QS stays in the accumulators; D_P KS goes to LDS.
//  Phase B  R = D_beta (V - D_P KS), lane = value column.
//  Phase C  finite Neumann recursion of Eq. 8: Z <- -G Z, U += Z for d_b steps.
//           Only structurally nonzero work is issued: at step m a row i needs
//           depth(i) >= m+1 and a column j must be a strict ancestor of i with
//           depth(j) >= m (Z^(m) vanishes on shallower rows).  G and C rows are
//           held in registers (lane j holds entry j of the row) and broadcast
//           with readlane; Z and U live in LDS, one column per lane, so no
//           access conflicts and no cross-lane traffic.
//  Phase D  readout O = B0 + C U, compact U written as float32.
#include "common.h"

namespace bole {

constexpr int kBV = 64;            // value columns per workgroup
constexpr int kLds = kBV + 4;      // padded LDS row (floats)
constexpr int kSlots = kMaxTree / 4;  // node rows owned per wave (node i -> wave i % 4)

template <int DT>
__device__ __forceinline__ void load_a8(const void* base, int64_t elem, bool ok, bf16x8& hi,
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
__device__ __forceinline__ float load_scalar(const void* base, int64_t elem) {
  if (DT == BOLE_BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(base)[elem]);
  return reinterpret_cast<const float*>(base)[elem];
}

template <int DT>
__device__ __forceinline__ void store_scalar(void* base, int64_t elem, float x) {
  if (DT == BOLE_BF16)
    reinterpret_cast<uint16_t*>(base)[elem] = float_to_bf16_bits(x);
  else
    reinterpret_cast<float*>(base)[elem] = x;
}

__device__ __forceinline__ float bcast(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int DT>
__global__ __launch_bounds__(256, 3) void verify_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ logP, const float* __restrict__ beta,
    const float* __restrict__ state_pool, int32_t n_slots, const int32_t* __restrict__ slot,
    const float* __restrict__ G, const float* __restrict__ C,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ depth,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ tree_depth, int32_t B,
    int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* __restrict__ O,
    float* __restrict__ U, uint32_t* __restrict__ err) {
  __shared__ float Za[kMaxTree * kLds];
  __shared__ float Zb[kMaxTree * kLds];
  __shared__ float Ub[kMaxTree * kLds];

  const int NV = (d_v + kBV - 1) / kBV;
  const int lid = xcd_remap(blockIdx.x, B * H * NV);
  const int unit = lid / NV, r = lid - (lid / NV) * NV;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform

  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (threadIdx.x == 0 && h == 0 && r == 0) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  const int td = tree_depth[b];
  if (td < 0) return;  // rejected by tree preparation
  const int s = slot[b];
  if (s < 0 || s >= n_slots) {
    if (threadIdx.x == 0 && h == 0 && r == 0) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int d_b = min(td, T - 1);

  // per-node topology, lane l <-> node l
  const bool nlive = lane < T;
  const int ndep = nlive ? depth[off + lane] : -1;
  const uint64_t nanc = nlive ? anc[off + lane] : 0ull;

  // G and C rows of this wave's nodes (node i = 4t + w), lane j holds entry j
  const float* Gt = G + (int64_t)unit * kMaxTree * kMaxTree;
  const float* Ct = C + (int64_t)unit * kMaxTree * kMaxTree;
  float grow[kSlots], crow[kSlots];
#pragma unroll
  for (int t = 0; t < kSlots; ++t) {
    const int i = 4 * t + w;
    grow[t] = i < T ? Gt[i * kMaxTree + lane] : 0.0f;
    crow[t] = i < T ? Ct[i * kMaxTree + lane] : 0.0f;
  }

  // ---------------- Phase A: [Q;K] S_pre^(r) on MFMA ----------------
  const int vloc = 16 * w + (lane & 15);
  const int vcol = kBV * r + vloc;
  const bool vin = vcol < d_v;
  const float* Srow = state_pool + (((int64_t)s * H + h) * d_v + (vin ? vcol : 0)) * d_k;
  const int kgrp = 8 * (lane >> 4);
  const int nmt = (T + 15) >> 4;
  f32x4 qs[4], ks[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    qs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    ks[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int kc = 0; kc < d_k; kc += 32) {
    const int kidx = kc + kgrp;
    const bool kin = kidx < d_k;
    float sx[8];
    if (vin && kin) {
      load_f32x8(Srow + kidx, sx);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) sx[e] = 0.0f;
    }
    bf16x8 b_hi, b_lo;
    split_bf16x8(sx, b_hi, b_lo);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nmt) {
        const int row = 16 * mt + (lane & 15);
        const bool ok = row < T && kin;
        const int64_t e = ((int64_t)(off + (ok ? row : 0)) * H + h) * d_k + kidx;
        bf16x8 aq_hi, aq_lo, ak_hi, ak_lo;
        load_a8<DT>(q, e, ok, aq_hi, aq_lo);
        load_a8<DT>(k, e, ok, ak_hi, ak_lo);
        qs[mt] = mfma_bf16(aq_hi, b_hi, qs[mt]);
        qs[mt] = mfma_bf16(aq_hi, b_lo, qs[mt]);
        ks[mt] = mfma_bf16(ak_hi, b_hi, ks[mt]);
        ks[mt] = mfma_bf16(ak_hi, b_lo, ks[mt]);
        if (DT == BOLE_F32) {
          qs[mt] = mfma_bf16(aq_lo, b_hi, qs[mt]);
          ks[mt] = mfma_bf16(ak_lo, b_hi, ks[mt]);
        }
      }
    }
  }
  // B0 = D_P QS (kept in registers), D_P KS -> LDS
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + 4 * (lane >> 4) + e;
        if (i < T) {
          const float P = expf(logP[(int64_t)(off + i) * H + h]);
          qs[mt][e] *= P;
          Za[i * kLds + vloc] = P * ks[mt][e];
        }
      }
    }
  }
  __syncthreads();

  // ---------------- Phase B: R = D_beta (V - D_P K S) ----------------
  const int c = lane;
  const int col = kBV * r + c;
  const bool cin = col < d_v;
  for (int i = w; i < T; i += 4) {
    const int64_t tok = (int64_t)(off + i) * H + h;
    const float vv = cin ? load_scalar<DT>(v, tok * d_v + col) : 0.0f;
    const float R = beta[tok] * (vv - Za[i * kLds + c]);
    Za[i * kLds + c] = R;
    Ub[i * kLds + c] = R;
  }
  __syncthreads();

  // ---------------- Phase C: Neumann recursion (Eq. 8) ----------------
  float* zc = Za;
  float* zn = Zb;
  for (int m = 0; m < d_b; ++m) {
    const uint64_t cols = ballot64(ndep >= m);
#pragma unroll
    for (int t = 0; t < kSlots; ++t) {
      const int i = 4 * t + w;
      if (i < T) {
        const int di = __builtin_amdgcn_readlane(ndep, i);
        if (di >= m + 1) {
          const uint32_t alo = __builtin_amdgcn_readlane((uint32_t)nanc, i);
          const uint32_t ahi = __builtin_amdgcn_readlane((uint32_t)(nanc >> 32), i);
          uint64_t pm = (((uint64_t)ahi << 32) | alo) & cols & ~(1ull << i);
          float acc0 = 0.0f, acc1 = 0.0f;
          while (pm) {
            const int j0 = __builtin_ctzll(pm);
            pm &= pm - 1;
            acc0 = fmaf(bcast(grow[t], j0), zc[j0 * kLds + c], acc0);
            if (pm) {
              const int j1 = __builtin_ctzll(pm);
              pm &= pm - 1;
              acc1 = fmaf(bcast(grow[t], j1), zc[j1 * kLds + c], acc1);
            }
          }
          const float z = -(acc0 + acc1);
          zn[i * kLds + c] = z;
          Ub[i * kLds + c] += z;
        }
      }
    }
    __syncthreads();
    float* tmp = zc;
    zc = zn;
    zn = tmp;
  }

  // ---------------- Phase D: readout O = B0 + C U ----------------
#pragma unroll
  for (int t = 0; t < kSlots; ++t) {
    const int i = 4 * t + w;
    if (i < T) {
      const uint32_t alo = __builtin_amdgcn_readlane((uint32_t)nanc, i);
      const uint32_t ahi = __builtin_amdgcn_readlane((uint32_t)(nanc >> 32), i);
      uint64_t pm = ((uint64_t)ahi << 32) | alo;
      float acc0 = 0.0f, acc1 = 0.0f;
      while (pm) {
        const int j0 = __builtin_ctzll(pm);
        pm &= pm - 1;
        acc0 = fmaf(bcast(crow[t], j0), Ub[j0 * kLds + c], acc0);
        if (pm) {
          const int j1 = __builtin_ctzll(pm);
          pm &= pm - 1;
          acc1 = fmaf(bcast(crow[t], j1), Ub[j1 * kLds + c], acc1);
        }
      }
      const int64_t tok = (int64_t)(off + i) * H + h;
      if (cin) U[tok * d_v + col] = Ub[i * kLds + c];
      zn[i * kLds + c] = acc0 + acc1;
    }
  }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + 4 * (lane >> 4) + e;
        if (i < T) zn[i * kLds + vloc] += qs[mt][e];
      }
    }
  }
  __syncthreads();
  for (int i = w; i < T; i += 4) {
    const int64_t tok = (int64_t)(off + i) * H + h;
    if (cin) store_scalar<DT>(O, tok * d_v + col, zn[i * kLds + c]);
  }
}

}  // namespace bole

extern "C" int bole_verify_launch(int32_t dtype, const void* q, const void* k, const void* v,
                                  const float* logP, const float* beta, const float* state_pool,
                                  int32_t n_slots, const int32_t* slot, const float* G,
                                  const float* C, const uint64_t* anc, const int32_t* depth,
                                  const int32_t* tree_off, const int32_t* tree_depth, int32_t B,
                                  int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O,
                                  float* U, uint32_t* err, hipStream_t s) {
  const int NV = (d_v + bole::kBV - 1) / bole::kBV;
  const dim3 grid(B * H * NV), block(256);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::verify_kernel<BOLE_BF16>, grid, block, 0, s, q, k, v, logP, beta,
                       state_pool, n_slots, slot, G, C, anc, depth, tree_off, tree_depth, B, N,
                       H, d_k, d_v, O, U, err);
  else
    hipLaunchKernelGGL(bole::verify_kernel<BOLE_F32>, grid, block, 0, s, q, k, v, logP, beta,
                       state_pool, n_slots, slot, G, C, anc, depth, tree_off, tree_depth, B, N,
                       H, d_k, d_v, O, U, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
