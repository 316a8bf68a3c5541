// Round-level topology step and log-space gate products.
//
// Topology (arXiv page of Bole: ancestor mask; review, Lemma 3's depth d):
// one wave64 per tree, one lane per node.  The ancestor-or-self set is built
// by pointer jumping: after round s every lane knows the first 2^s nodes of
// its upward path and the node 2^s steps up; six rounds cover any path of a
// tree with at most 64 nodes, so a lane that still has a jump target after six
// rounds lies on or leads into a cycle.
//
// Gate products (review, Eq. 4 paragraph: P_i multiplies the gates of i's
// ancestors and of i): logP_i = logP_parent(i) + g_i in float32, evaluated in
// level order so every parent is final before its children, which makes each
// value the root-first running sum of g along the path.
#include "common.h"

namespace bole {

__global__ __launch_bounds__(64) void tree_topology_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tree_off, int32_t N,
    int32_t* __restrict__ depth_out, uint64_t* __restrict__ anc_out,
    int32_t* __restrict__ order_out, int32_t* __restrict__ tree_depth_out,
    uint32_t* __restrict__ err) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (lane == 0) {
      tree_depth_out[b] = -1;
      report(err, BOLE_ERR_TREE_SIZE);
    }
    return;
  }
  const bool live = lane < T;
  const int p = live ? parent[off + lane] : -1;
  const bool bad = live && p != -1 && (p < 0 || p >= T || p == lane);
  if (ballot64(bad)) {
    if (lane == 0) {
      tree_depth_out[b] = -1;
      report(err, BOLE_ERR_BAD_PARENT);
    }
    return;
  }
  uint64_t anc = live ? (1ull << lane) : 0ull;
  int jmp = live ? p : -1;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    const int src = jmp >= 0 ? jmp : lane;
    const uint64_t a2 = __shfl(anc, src);
    const int j2 = __shfl(jmp, src);
    if (jmp >= 0) {
      anc |= a2;
      jmp = j2;
    }
  }
  if (ballot64(live && jmp >= 0)) {
    if (lane == 0) {
      tree_depth_out[b] = -1;
      report(err, BOLE_ERR_CYCLE);
    }
    return;
  }
  const int dep = live ? __popcll(anc) - 1 : -1;
  int dmax = dep;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) dmax = max(dmax, __shfl_xor(dmax, s));
  // stable sort by (depth, local id): rank = nodes on shallower levels plus
  // lower ids on the same level
  int base = 0, pos = 0;
  for (int lev = 0; lev <= dmax; ++lev) {
    const uint64_t m = ballot64(dep == lev);
    if (dep == lev) pos = base + __popcll(m & ((1ull << lane) - 1ull));
    base += __popcll(m);
  }
  if (live) {
    depth_out[off + lane] = dep;
    anc_out[off + lane] = anc;
    order_out[off + pos] = lane;
  }
  if (lane == 0) tree_depth_out[b] = dmax;
}

// grid (B, ceil(L*H / 64)); thread -> one (layer, head) column of one tree.
__global__ __launch_bounds__(64) void gate_logp_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tree_off,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tree_depth, int32_t N,
    int32_t L, int32_t H, const float* __restrict__ g, float* __restrict__ logP) {
  __shared__ float val[kMaxTree][64];
  const int b = blockIdx.x;
  if (tree_depth[b] < 0) return;
  const int off = tree_off[b];
  const int T = tree_off[b + 1] - off;
  const int lh = blockIdx.y * 64 + threadIdx.x;
  if (lh >= L * H) return;
  const int l = lh / H, h = lh - (lh / H) * H;
  const int64_t base = (int64_t)l * N * H + h;
  for (int p = 0; p < T; ++p) {
    const int i = order[off + p];
    const int par = parent[off + i];
    const float prev = par < 0 ? 0.0f : val[par][threadIdx.x];
    const float x = __fadd_rn(prev, g[base + (int64_t)(off + i) * H]);
    val[i][threadIdx.x] = x;
    logP[base + (int64_t)(off + i) * H] = x;
  }
}

}  // namespace bole

extern "C" int bole_tree_prep_launch(const int32_t* parent, const int32_t* tree_off, int32_t B,
                                     int32_t N, const float* log_gamma, int32_t L, int32_t H,
                                     int32_t* depth, uint64_t* anc, int32_t* order,
                                     int32_t* tree_depth, float* logP, uint32_t* err,
                                     hipStream_t s) {
  hipLaunchKernelGGL(bole::tree_topology_kernel, dim3(B), dim3(64), 0, s, parent, tree_off, N,
                     depth, anc, order, tree_depth, err);
  if (hipGetLastError() != hipSuccess) return BOLE_E_HIP;
  if (log_gamma) {
    const int cols = L * H;
    hipLaunchKernelGGL(bole::gate_logp_kernel, dim3(B, (cols + 63) / 64), dim3(64), 0, s, parent,
                       tree_off, order, tree_depth, N, L, H, log_gamma, logP);
    if (hipGetLastError() != hipSuccess) return BOLE_E_HIP;
  }
  return BOLE_OK;
}
