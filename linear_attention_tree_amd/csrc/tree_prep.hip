// Round-level topology step and log-space gate products.
//
// Topology: one wave64 per tree, one lane per node (tree_topo.h).
//
// Gate products (review, Eq. 4 paragraph: P_i multiplies the gates of i's
// ancestors and of i): logP_i is the root-first running sum of g along the path
// in float32, one rounding per add (so logP_i = logP_parent(i) + g_i exactly as
// computed for the parent).
#include "tree_topo.h"

namespace bole {

constexpr int kGateCols = 64;    // (layer, head) columns per workgroup
constexpr int kPrepThreads = 256;
constexpr int kColsPerThread = 16;
constexpr int kValStride = kGateCols + 4;  // floats per LDS row: 16-byte aligned, rows 4 banks apart

// grid (B, max(1, ceil(L*H / 64))).  Thread t owns node t/4 of the tree and 16
// consecutive (layer, head) columns of the block.  Wave 0 derives the tree's
// topology (every column block does; block row 0 publishes it) and a path
// table, path[i][d] = the ancestor of i at depth d, while all threads fetch
// their gates.  Each node's logP is then its own root-first sum along the path
// table: the same float32 additions, in the same order, as a level-by-level
// sweep, with no barrier per level.
__global__ __launch_bounds__(kPrepThreads) void tree_prep_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tree_off, int32_t N,
    int32_t L, int32_t H, const float* __restrict__ g, int32_t* __restrict__ depth_out,
    uint64_t* __restrict__ anc_out, int32_t* __restrict__ order_out,
    int32_t* __restrict__ tree_depth_out, float* __restrict__ logP, int32_t vec,
    uint32_t* __restrict__ err) {
  __shared__ __align__(16) float val[kMaxTree * kValStride];
  __shared__ uint8_t path[kMaxTree][kMaxTree];
  __shared__ int node_dep[kMaxTree];
  __shared__ int tree_ok;
  const int b = blockIdx.x;
  const bool publish = blockIdx.y == 0;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  const bool size_ok = !(off < 0 || end > N || T < 1 || T > kMaxTree);
  if (!size_ok) {
    if (threadIdx.x == 0 && publish) {
      tree_depth_out[b] = -1;
      report(err, BOLE_ERR_TREE_SIZE);
    }
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // wave 0's parent loads go out first: the topology chain starts from them
  int p = -1;
  if (w == 0) p = parent[off + min(lane, T - 1)];

  // gate values of this thread's node and columns, every load in flight
  // together (a node past the tree reads node T-1 and a column group past L*H
  // reads group 0; neither is stored)
  const int i = threadIdx.x >> 2;
  const int c0 = kColsPerThread * (threadIdx.x & 3);
  const int lh0 = blockIdx.y * kGateCols + c0;
  const int LH = L * H;
  // vec (host-checked): H % 16 == 0 and g, logP 16-byte aligned, so a thread's
  // 16 columns are one layer's contiguous, aligned float4s
  const int ic = min(i, T - 1);
  float gv[kColsPerThread];
  if (g != nullptr) {  // uniform
    if (vec) {
      const int lhc = lh0 < LH ? lh0 : 0;
      const int l = lhc / H, h0 = lhc - (lhc / H) * H;
      const f32x4* src =
          reinterpret_cast<const f32x4*>(g + ((int64_t)l * N + off + ic) * H + h0);
#pragma unroll
      for (int q = 0; q < kColsPerThread / 4; ++q) {
        const f32x4 x = src[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[4 * q + e] = x[e];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int lh = lh0 + k < LH ? lh0 + k : 0;
        const int l = lh / H, h = lh - (lh / H) * H;
        gv[k] = g[((int64_t)l * N + off + ic) * H + h];
      }
    }
  }

  if (w == 0) {
    const TreeTopo tp = tree_topology(lane, T, p);
    const uint32_t fail = tp.fail;
    const int dmax = tp.dmax;
    if (!fail) {
      if (lane < T) {
        node_dep[lane] = tp.dep;
        if (publish) {
          depth_out[off + lane] = tp.dep;
          anc_out[off + lane] = tp.anc;
          order_out[off + tp.pos] = lane;
        }
        // path table: every ancestor-or-self j of this node at its depth
        uint64_t m = tp.anc;
        while (m) {
          const int j = __builtin_ctzll(m);
          path[lane][node_dep[j]] = (uint8_t)j;
          m &= m - 1ull;
        }
      }
    }
    if (lane == 0) {
      tree_ok = fail == 0;
      if (publish) {
        tree_depth_out[b] = fail ? -1 : dmax;
        if (fail) report(err, fail);
      }
    }
  }
  if (g != nullptr && i < T) {
#pragma unroll
    for (int q = 0; q < kColsPerThread / 4; ++q)
      *reinterpret_cast<f32x4*>(val + i * kValStride + c0 + 4 * q) =
          f32x4{gv[4 * q], gv[4 * q + 1], gv[4 * q + 2], gv[4 * q + 3]};
  }
  __syncthreads();
  if (!tree_ok || g == nullptr) return;  // uniform over the workgroup
  if (i >= T) return;  // no barrier follows
  // root-first running sum along the path: starts at +0.0f, one rounding per add
  float acc[kColsPerThread];
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) acc[k] = 0.0f;
  const int di = node_dep[i];
  for (int d = 0; d <= di; ++d) {
    const f32x4* row = reinterpret_cast<const f32x4*>(val + path[i][d] * kValStride + c0);
#pragma unroll
    for (int q = 0; q < kColsPerThread / 4; ++q) {
      const f32x4 x = row[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * q + e] = __fadd_rn(acc[4 * q + e], x[e]);
    }
  }
  if (vec) {
    if (lh0 < LH) {
      const int l = lh0 / H, h0 = lh0 - (lh0 / H) * H;
      f32x4* dst = reinterpret_cast<f32x4*>(logP + ((int64_t)l * N + off + i) * H + h0);
#pragma unroll
      for (int q = 0; q < kColsPerThread / 4; ++q)
        dst[q] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  } else {
#pragma unroll
    for (int k = 0; k < kColsPerThread; ++k) {
      const int lh = lh0 + k;
      if (lh < LH) {
        const int l = lh / H, h = lh - (lh / H) * H;
        logP[((int64_t)l * N + off + i) * H + h] = acc[k];
      }
    }
  }
}

}  // namespace bole

extern "C" int bole_tree_prep_launch(const int32_t* parent, const int32_t* tree_off, int32_t B,
                                     int32_t N, const float* log_gamma, int32_t L, int32_t H,
                                     int32_t* depth, uint64_t* anc, int32_t* order,
                                     int32_t* tree_depth, float* logP, uint32_t* err,
                                     hipStream_t s) {
  const int cols = log_gamma ? L * H : 0;
  const int chunks = cols > 0 ? (cols + bole::kGateCols - 1) / bole::kGateCols : 1;
  const bool aligned = ((uintptr_t)log_gamma % 16 == 0) && ((uintptr_t)logP % 16 == 0);
  const int vec = H % bole::kColsPerThread == 0 && aligned;
  hipLaunchKernelGGL(bole::tree_prep_kernel, dim3(B, chunks), dim3(bole::kPrepThreads), 0, s,
                     parent, tree_off, N, L, H, log_gamma, depth, anc, order, tree_depth, logP,
                     vec, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
