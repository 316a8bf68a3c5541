// Tree-parallel short causal convolution: the first per-layer stage of the
// fused tree pipeline (arXiv page of Bole, section IV-C; review page, fused
// pipeline paragraph).  Each node's window is gathered by following its
// parents; the taps, the bias and SiLU are applied in the same pass, and the
// nodes are independent of one another.  The GDN layer's depthwise causal
// convolution (arXiv page, section II-A) sees, at node i, the last W entries of
// the request's committed conv state (the W - 1 inputs that preceded the tree,
// oldest first) followed by the inputs along i's root-to-node path: exactly
// what ordinary decoding of that path would see.
//
// y[i][c] = silu(bias[c] + sum_j weight[c][j] * window_i[j][c]), tap W-1 on
// node i's own input.  float32 arithmetic (SiLU on the hardware exp2 and
// reciprocal), output in the token dtype.
//
// The commit moves the accepted path's last W - 1 inputs into the request's
// conv state, in place.
#include <type_traits>

#include "tree_topo.h"

namespace bole {

constexpr int kMaxConv = 8;        // widest convolution supported
constexpr int kConvThreads = 256;

template <int DT, int WD = kMaxConv>
struct ConvCfg {
  using Elem = std::conditional_t<DT == BOLE_BF16, uint16_t, float>;
  static constexpr int EPP = 16 / sizeof(Elem);              // elements per 16-byte piece
  static constexpr int CH = DT == BOLE_BF16 ? 256 : 128;      // channels per workgroup (512 B)
  static constexpr int GROUPS = CH / EPP;                    // pieces per row
  static constexpr int NQ = 1;                               // parts taken in turn
  static constexpr int HG = GROUPS / NQ;                     // pieces per row and part
  static constexpr int NODE_LANES = kConvThreads / HG;       // nodes computed at once
  // 16-byte pieces per thread and part: tree rows plus committed state rows
  static constexpr int PIECES = (kMaxTree + WD - 1) * HG / kConvThreads + 1;
};

__device__ __forceinline__ float elem_to_float(uint16_t b) { return bf16_bits_to_float(b); }
__device__ __forceinline__ float elem_to_float(float f) { return f; }

// grid (B, ceil(C / CH)).  Rows 0..T-1 of the LDS tile hold the tree's inputs
// for the workgroup's channels, rows kMaxTree .. kMaxTree + WD - 2 the
// committed conv state.  src[i][j] is the tile row of the j-th most recent entry
// of node i's window (j = 0: node i itself).
//
// The width WD is a compile-time constant (the host picks the instantiation):
// a thread holds exactly WD taps per channel in registers, and the tile has
// exactly WD - 1 state rows, so narrow convolutions keep more workgroups
// resident.
//
// The workgroup's channels can be taken in NQ parts: a part's loads go out
// once the part before it has arrived, and the part before it is then computed
// and stored while they are in flight, so the output writes of one part
// overlap the input reads of the next.  With the width a compile-time constant
// (111 registers at W = 4 in bf16, against 159 for a kernel holding every
// width), one part measures faster at the target (13.2-13.7 us against
// 13.9-14.1 us for two), so NQ = 1: every load goes out at once.
template <int DT, int WD>
__global__ __launch_bounds__(kConvThreads) void tree_conv_kernel(
    const void* __restrict__ x, const float* __restrict__ weight, const float* __restrict__ bias,
    const void* __restrict__ conv_state, int32_t n_slots, const int32_t* __restrict__ slot,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tree_off, int32_t N, int32_t C,
    void* __restrict__ y, uint32_t* __restrict__ err) {
  using CC = ConvCfg<DT, WD>;
  using Elem = typename CC::Elem;
  constexpr int Wd = WD;
  __shared__ __align__(16) Elem tile[kMaxTree + WD - 1][CC::CH];
  __shared__ float ws[WD][CC::CH];
  __shared__ float bs[CC::CH];
  __shared__ int8_t src[kMaxTree][WD];
  __shared__ int tree_ok;

  const int b = blockIdx.x;
  const int c0 = CC::CH * blockIdx.y;
  const bool reporter = threadIdx.x == 0 && blockIdx.y == 0;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (reporter) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  const int s = Wd > 1 ? slot[b] : 0;
  if (Wd > 1 && (s < 0 || s >= n_slots)) {
    if (reporter) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const Elem* xe = reinterpret_cast<const Elem*>(x);
  const Elem* se = reinterpret_cast<const Elem*>(conv_state);

  // Wave 0's parent links go out first (the topology below waits only for
  // them), then each thread's pieces of part 0 of the tree's input rows and of
  // the committed state rows, then the taps.  A piece past the rows needed or
  // past C reads piece 0 of row 0 and is not stored.
  int p = -1;
  if (w == 0) p = parent[off + min(lane, T - 1)];
  const int n_pieces = (T + Wd - 1) * CC::HG;
  auto piece = [&](int h, int k, int& r, int& col) {  // tile row and column of a piece
    const int id = threadIdx.x + kConvThreads * k;
    r = id / CC::HG;
    col = CC::EPP * (CC::HG * h + (id - (id / CC::HG) * CC::HG));
    return id < n_pieces && c0 + col < C;
  };
  u16x8 buf[CC::NQ][CC::PIECES];
  auto issue = [&](auto h_tag) {
    constexpr int h = decltype(h_tag)::value;
#pragma unroll
    for (int k = 0; k < CC::PIECES; ++k) {
      int r, col;
      const bool use = piece(h, k, r, col);
      const Elem* row = !use ? xe : r < T ? xe + (int64_t)(off + r) * C
                                          : se + ((int64_t)s * (Wd - 1) + (r - T)) * C;
      buf[h][k] = *reinterpret_cast<const u16x8*>(row + (use ? c0 + col : 0));
    }
  };
  issue(std::integral_constant<int, 0>{});
  constexpr int kWPer = (WD * CC::CH + kConvThreads - 1) / kConvThreads;
  float wv[kWPer];
#pragma unroll
  for (int k = 0; k < kWPer; ++k) {
    const int id = threadIdx.x + kConvThreads * k;
    const int j = id / CC::CH, c = id - (id / CC::CH) * CC::CH;
    const bool use = j < Wd && c0 + c < C;
    wv[k] = weight[use ? (int64_t)(c0 + c) * Wd + j : 0];
  }
  const int cb = min(c0 + (int)threadIdx.x, C - 1);
  const float bv = bias != nullptr ? bias[cb] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);

  if (w == 0) {
    const TreeTopo tp = tree_topology(lane, T, p);
    if (!tp.fail && lane < T) {
      // walk up: entry j is the j-th ancestor while the path lasts, then the
      // committed state from its newest row backwards (the shuffles read
      // parents of tree nodes, all active lanes)
      int cur = lane;
      for (int j = 0; j < Wd; ++j) {
        src[lane][j] = (int8_t)(j <= tp.dep ? cur : kMaxTree + (Wd - 1) - (j - tp.dep));
        const int up = __shfl(p, max(cur, 0));
        cur = j < tp.dep ? up : -1;
      }
    }
    if (lane == 0) {
      tree_ok = !tp.fail;
      if (tp.fail && reporter) report(err, tp.fail);
    }
  }
  auto park = [&](auto h_tag) {  // waits for part h's pieces
    constexpr int h = decltype(h_tag)::value;
#pragma unroll
    for (int k = 0; k < CC::PIECES; ++k) {
      int r, col;
      if (piece(h, k, r, col))
        *reinterpret_cast<u16x8*>(&tile[r < T ? r : kMaxTree + r - T][col]) = buf[h][k];
    }
  };
  park(std::integral_constant<int, 0>{});
#pragma unroll
  for (int k = 0; k < kWPer; ++k) {
    const int id = threadIdx.x + kConvThreads * k;
    if (id < WD * CC::CH) ws[id / CC::CH][id - (id / CC::CH) * CC::CH] = wv[k];
  }
  if (threadIdx.x < CC::CH) bs[threadIdx.x] = c0 + (int)threadIdx.x < C ? bv : 0.0f;
  __syncthreads();  // part 0, taps, bias and the window table visible
  if (!tree_ok) return;  // uniform

  const int pc = threadIdx.x % CC::HG, nl = threadIdx.x / CC::HG;
  auto half = [&](auto h_tag) {
    constexpr int h = decltype(h_tag)::value;
    const int cl = CC::EPP * (CC::HG * h + pc), c = c0 + cl;
    if (c >= C) return;
    Elem* ye = reinterpret_cast<Elem*>(y) + c;
    // the thread's taps and bias stay in registers across its nodes
    float wr[WD][CC::EPP], br[CC::EPP];
#pragma unroll
    for (int e = 0; e < CC::EPP; ++e) {
      br[e] = bs[cl + e];
#pragma unroll
      for (int j = 0; j < WD; ++j) wr[j][e] = ws[j][cl + e];
    }
    for (int i = nl; i < T; i += CC::NODE_LANES) {
      float acc[CC::EPP];
#pragma unroll
      for (int e = 0; e < CC::EPP; ++e) acc[e] = br[e];
#pragma unroll
      for (int j = 0; j < WD; ++j) {  // j-th most recent entry, tap WD-1-j
        const u16x8 raw = *reinterpret_cast<const u16x8*>(&tile[src[i][j]][cl]);
        const Elem* v = reinterpret_cast<const Elem*>(&raw);
#pragma unroll
        for (int e = 0; e < CC::EPP; ++e) acc[e] = fmaf(wr[WD - 1 - j][e], elem_to_float(v[e]), acc[e]);
      }
      u16x8 out;
      Elem* o = reinterpret_cast<Elem*>(&out);
#pragma unroll
      for (int e = 0; e < CC::EPP; ++e) {
        // SiLU a / (1 + e^-a) on the hardware exp2 and reciprocal (relative
        // error near 1e-6 for |a| < 100; e^-a overflows to inf, giving -0, for
        // very negative a)
        const float a = acc[e];
        const float sv = a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
        if constexpr (DT == BOLE_BF16)
          o[e] = float_to_bf16_bits(sv);
        else
          o[e] = sv;
      }
      // streamed out: the outputs are not read again by this kernel
      __builtin_nontemporal_store(out, reinterpret_cast<u16x8*>(ye + (int64_t)(off + i) * C));
    }
  };
  auto compute = [&](auto h_tag) { half(h_tag); };
  auto stage = [&](auto h_tag, auto self) {
    constexpr int h = decltype(h_tag)::value;
    if constexpr (h + 1 < CC::NQ) {
      issue(std::integral_constant<int, h + 1>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    compute(h_tag);
    if constexpr (h + 1 < CC::NQ) {
      park(std::integral_constant<int, h + 1>{});
      __syncthreads();  // part h + 1 visible (other parts' columns are not touched)
      self(std::integral_constant<int, h + 1>{}, self);
    }
  };
  stage(std::integral_constant<int, 0>{}, stage);
}

// grid (B, ceil(C / 256)); thread = channel.  Reads every source of the new
// state before writing any of it (the update is in place).
template <int DT>
__global__ __launch_bounds__(kConvThreads) void conv_commit_kernel(
    void* __restrict__ conv_state, int32_t n_slots, const int32_t* __restrict__ slot,
    const void* __restrict__ x, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t N, int32_t C,
    int32_t Wd, uint32_t* __restrict__ err) {
  using Elem = typename ConvCfg<DT>::Elem;
  __shared__ int srcs[kMaxConv];  // >= 0: tree node; < 0: -1 - (old state row)
  __shared__ int tree_ok;
  const int b = blockIdx.x;
  const int a = accept[b];
  if (a == -1 || Wd < 2) return;
  const bool reporter = threadIdx.x == 0 && blockIdx.y == 0;
  const int off = tree_off[b], end = tree_off[b + 1];
  const int T = end - off;
  if (off < 0 || end > N || T < 1 || T > kMaxTree) {
    if (reporter) report(err, BOLE_ERR_TREE_SIZE);
    return;
  }
  if (a < 0 || a >= T) {
    if (reporter) report(err, BOLE_ERR_BAD_ACCEPT);
    return;
  }
  const int s = slot[b];
  if (s < 0 || s >= n_slots) {
    if (reporter) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w == 0) {
    const int p = parent[off + min(lane, T - 1)];
    const TreeTopo tp = tree_topology(lane, T, p);
    if (!tp.fail) {
      // new row k (oldest first) is the (W-2-k)-th most recent entry of the
      // accepted path's window
      const int da = __shfl(tp.dep, a);
      int cur = a;
      for (int j = 0; j < Wd - 1; ++j) {
        if (lane == 0) srcs[Wd - 2 - j] = j <= da ? cur : -1 - ((Wd - 1) - (j - da));
        const int up = __shfl(p, max(cur, 0));
        cur = j < da ? up : -1;
      }
    }
    if (lane == 0) {
      tree_ok = !tp.fail;
      if (tp.fail && reporter) report(err, tp.fail);
    }
  }
  __syncthreads();
  if (!tree_ok) return;
  const int c = 256 * blockIdx.y + threadIdx.x;
  if (c >= C) return;
  Elem* st = reinterpret_cast<Elem*>(conv_state) + (int64_t)s * (Wd - 1) * C + c;
  const Elem* xe = reinterpret_cast<const Elem*>(x) + c;
  Elem vals[kMaxConv];
#pragma unroll
  for (int k = 0; k < kMaxConv - 1; ++k) {
    if (k < Wd - 1) {
      const int sr = srcs[k];
      vals[k] = sr >= 0 ? xe[(int64_t)(off + sr) * C] : st[(int64_t)(-1 - sr) * C];
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxConv - 1; ++k)
    if (k < Wd - 1) st[(int64_t)k * C] = vals[k];
}

}  // namespace bole

extern "C" int bole_tree_conv_launch(int32_t dtype, const void* x, const float* weight,
                                     const float* bias, const void* conv_state, int32_t n_slots,
                                     const int32_t* slot, const int32_t* parent,
                                     const int32_t* tree_off, int32_t B, int32_t N, int32_t C,
                                     int32_t W, void* y, uint32_t* err, hipStream_t s) {
  const dim3 block(bole::kConvThreads);
  auto go = [&](auto dt_tag, auto w_tag) {
    constexpr int DT = decltype(dt_tag)::value, WD = decltype(w_tag)::value;
    using CC = bole::ConvCfg<DT, WD>;
    const dim3 grid(B, (C + CC::CH - 1) / CC::CH);
    hipLaunchKernelGGL((bole::tree_conv_kernel<DT, WD>), grid, block, 0, s, x, weight, bias,
                       conv_state, n_slots, slot, parent, tree_off, N, C, y, err);
  };
  auto by_width = [&](auto dt_tag) {
    switch (W) {  // 1 .. kMaxConv, checked by the caller
      case 1: go(dt_tag, std::integral_constant<int, 1>{}); break;
      case 2: go(dt_tag, std::integral_constant<int, 2>{}); break;
      case 3: go(dt_tag, std::integral_constant<int, 3>{}); break;
      case 4: go(dt_tag, std::integral_constant<int, 4>{}); break;
      case 5: go(dt_tag, std::integral_constant<int, 5>{}); break;
      case 6: go(dt_tag, std::integral_constant<int, 6>{}); break;
      case 7: go(dt_tag, std::integral_constant<int, 7>{}); break;
      default: go(dt_tag, std::integral_constant<int, 8>{}); break;
    }
  };
  if (dtype == BOLE_BF16)
    by_width(std::integral_constant<int, BOLE_BF16>{});
  else
    by_width(std::integral_constant<int, BOLE_F32>{});
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}

extern "C" int bole_conv_commit_launch(int32_t dtype, void* conv_state, int32_t n_slots,
                                       const int32_t* slot, const void* x, const int32_t* parent,
                                       const int32_t* tree_off, const int32_t* accept, int32_t B,
                                       int32_t N, int32_t C, int32_t W, uint32_t* err,
                                       hipStream_t s) {
  const dim3 grid(B, (C + 255) / 256), block(bole::kConvThreads);
  if (dtype == BOLE_BF16)
    hipLaunchKernelGGL(bole::conv_commit_kernel<BOLE_BF16>, grid, block, 0, s, conv_state,
                       n_slots, slot, x, parent, tree_off, accept, N, C, W, err);
  else
    hipLaunchKernelGGL(bole::conv_commit_kernel<BOLE_F32>, grid, block, 0, s, conv_state,
                       n_slots, slot, x, parent, tree_off, accept, N, C, W, err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
