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
// ancestors and of i): logP_i = logP_parent(i) + g_i in float32, evaluated level
// by level so every parent is final before its children, which makes each value
// the root-first running sum of g along the path (one rounding per add).
#include "common.h"

namespace bole {

constexpr int kGateCols = 64;    // (layer, head) columns per workgroup
constexpr int kPrepThreads = 256;

// grid (B, max(1, ceil(L*H / 64))).  Wave 0 derives the tree's topology in LDS
// (every column block does, it is one wave of shuffles); block row 0 publishes
// it.  Meanwhile all waves fetch the gate values of the block's 64 columns, then
// sweep the levels in order, four node slots per column.
__global__ __launch_bounds__(kPrepThreads) void tree_prep_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tree_off, int32_t N,
    int32_t L, int32_t H, const float* __restrict__ g, int32_t* __restrict__ depth_out,
    uint64_t* __restrict__ anc_out, int32_t* __restrict__ order_out,
    int32_t* __restrict__ tree_depth_out, float* __restrict__ logP, uint32_t* __restrict__ err) {
  __shared__ float val[kMaxTree][kGateCols + 1];
  __shared__ int lvl_node[kMaxTree], lvl_par[kMaxTree], lvl_start[kMaxTree + 1];
  __shared__ int tree_ok, tree_dmax;
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
  // gate values of this block's columns (independent of the topology)
  const int c = threadIdx.x & (kGateCols - 1);
  const int lh = blockIdx.y * kGateCols + c;
  const bool col_ok = g != nullptr && lh < L * H;
  const int l = col_ok ? lh / H : 0, h = col_ok ? lh - (lh / H) * H : 0;
  const int64_t base = (int64_t)l * N * H + h;
  // every gate load is issued before the first is stored: node T-1 stands in
  // for slots past the tree and column (0, 0) for columns past L*H, neither of
  // which is stored
  if (g != nullptr) {  // uniform
    constexpr int kPer = kMaxTree / (kPrepThreads / 64);
    const float* gcol = g + base + (int64_t)off * H;  // node i at gcol[i * H]
    float gv[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) gv[r] = gcol[min(w + (kPrepThreads / 64) * r, T - 1) * H];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = w + (kPrepThreads / 64) * r;
      if (col_ok && i < T) val[i][c] = gv[r];
    }
  }

  if (w == 0) {
    const bool live = lane < T;
    p = live ? p : -1;
    const bool bad = live && p != -1 && (p < 0 || p >= T || p == lane);
    uint32_t fail = 0;
    int dmax = 0;
    if (ballot64(bad)) {
      fail = BOLE_ERR_BAD_PARENT;
    } else {
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
        fail = BOLE_ERR_CYCLE;
      } else {
        const int dep = live ? __popcll(anc) - 1 : -1;
        dmax = dep;
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1) dmax = max(dmax, __shfl_xor(dmax, sh));
        // stable sort by (depth, local id): rank = nodes on shallower levels plus
        // lower ids on the same level
        int acc = 0, pos = 0;
        for (int lev = 0; lev <= dmax; ++lev) {
          const uint64_t m = ballot64(dep == lev);
          if (dep == lev) pos = acc + __popcll(m & ((1ull << lane) - 1ull));
          if (lane == 0) lvl_start[lev] = acc;
          acc += __popcll(m);
        }
        if (lane == 0) lvl_start[dmax + 1] = T;
        if (live) {
          lvl_node[pos] = lane;
          lvl_par[pos] = p;
          if (publish) {
            depth_out[off + lane] = dep;
            anc_out[off + lane] = anc;
            order_out[off + pos] = lane;
          }
        }
      }
    }
    if (lane == 0) {
      tree_ok = fail == 0;
      tree_dmax = dmax;
      if (publish) {
        tree_depth_out[b] = fail ? -1 : dmax;
        if (fail) report(err, fail);
      }
    }
  }
  __syncthreads();
  if (!tree_ok || g == nullptr) return;  // uniform over the workgroup
  const int td = tree_dmax;
  // roots add their gate to +0.0f, every other node to its parent's finished sum
  for (int lev = 0; lev <= td; ++lev) {
    const int p0 = lvl_start[lev], p1 = lvl_start[lev + 1];
    for (int p = p0 + w; p < p1; p += kPrepThreads / 64) {
      const int i = lvl_node[p], par = lvl_par[p];
      const float prev = par < 0 ? 0.0f : val[par][c];
      val[i][c] = __fadd_rn(prev, val[i][c]);
    }
    __syncthreads();
  }
  if (col_ok) {
    float* lcol = logP + base + (int64_t)off * H;
    for (int i = w; i < T; i += kPrepThreads / 64) lcol[i * H] = val[i][c];
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
  hipLaunchKernelGGL(bole::tree_prep_kernel, dim3(B, chunks), dim3(bole::kPrepThreads), 0, s,
                     parent, tree_off, N, L, H, log_gamma, depth, anc, order, tree_depth, logP,
                     err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
