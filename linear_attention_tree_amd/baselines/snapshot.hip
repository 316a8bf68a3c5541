// The per-node full-state-snapshot verifier: the baseline tree verification
// the pages compare against (arXiv page, section V's verification-core
// comparison with SGLang-Tree's serial delta-rule verifier; section IV-D: a
// full d_k x d_v state per node and head).  It is a measurement baseline, not
// part of libbole's interface.
//
// Every node's state is materialised in HBM, level by level: one launch per
// tree depth, one workgroup per (node at that depth, head).  The workgroup reads
// its parent's state (the committed slot state for a root), applies one step
// of the GDN recurrence (Eq. 1 of the paper):
//     S~ = gamma S_parent;  u = beta (v - S~^T k);  S = S~ + k u^T;  o = S^T q
// and writes the node's full state, O and U.  The commit copies the accepted
// node's state into the slot.  float32 arithmetic; states use the slot layout
// [.., H, d_v, d_k] (row v holds S[:, v]).
//
// A workgroup of 256 threads takes 8 state rows at a time: each 32-lane half
// of a wave owns one row, each lane 4 consecutive keys of it per 128-key
// chunk, so a row moves as 512-byte coalesced pieces, read once and written
// once.  The two dot products of a row (S~^T k and S^T q) are butterfly sums
// within the half-wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerPass = kThreads / 32;
constexpr int kMaxChunks = 2;  // d_k <= 256: two 128-key chunks per row

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ float tok(const void* p, int64_t i) {
  if (BF16) return __uint_as_float(((uint32_t) reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  return reinterpret_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void put(void* p, int64_t i, float x) {
  if (BF16)
    reinterpret_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
  else
    reinterpret_cast<float*>(p)[i] = x;
}

__device__ __forceinline__ float half_wave_sum(float x) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) x += __shfl_xor(x, m, 32);
  return x;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void snapshot_level_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* __restrict__ state_pool, const int32_t* __restrict__ slot,
    const int32_t* __restrict__ node_tree, const int32_t* __restrict__ parent_node,
    const int32_t* __restrict__ level_nodes, float* __restrict__ snap, void* __restrict__ O,
    float* __restrict__ U, int32_t H, int32_t d_k, int32_t d_v) {
  const int li = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int node = level_nodes[li];
  const int par = parent_node[node];
  const int64_t sz = (int64_t)d_v * d_k;
  const float* Sp = par < 0 ? state_pool + ((int64_t)slot[node_tree[node]] * H + h) * sz
                            : snap + ((int64_t)par * H + h) * sz;
  float* Sd = snap + ((int64_t)node * H + h) * sz;
  const int64_t tk = (int64_t)node * H + h;
  const float gamma = expf(g[tk]), bt = beta[tk];
  const int lane32 = threadIdx.x & 31, row0 = threadIdx.x >> 5;
  // this lane's keys: 4 lane32 .. + 3 of each 128-key chunk
  f32x4 kr[kMaxChunks], qr[kMaxChunks];
  const int nch = (d_k + 127) / 128;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = 128 * c + 4 * lane32 + e;
      const bool in = c < nch && col < d_k;
      kr[c][e] = in ? tok<BF16>(k, tk * d_k + col) : 0.0f;
      qr[c][e] = in ? tok<BF16>(q, tk * d_k + col) : 0.0f;
    }
  }
  for (int r = row0; r < d_v; r += kRowsPerPass) {
    const float* src = Sp + (int64_t)r * d_k;
    float* dst = Sd + (int64_t)r * d_k;
    f32x4 s[kMaxChunks];
    float w = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int col = 128 * c + 4 * lane32;
      s[c] = c < nch && col < d_k ? *reinterpret_cast<const f32x4*>(src + col) * gamma
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
      w += s[c][0] * kr[c][0] + s[c][1] * kr[c][1] + s[c][2] * kr[c][2] + s[c][3] * kr[c][3];
    }
    w = half_wave_sum(w);
    const float u = bt * (tok<BF16>(v, tk * d_v + r) - w);
    float o = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int col = 128 * c + 4 * lane32;
      const f32x4 sn = s[c] + u * kr[c];
      if (c < nch && col < d_k) *reinterpret_cast<f32x4*>(dst + col) = sn;
      o += sn[0] * qr[c][0] + sn[1] * qr[c][1] + sn[2] * qr[c][2] + sn[3] * qr[c][3];
    }
    o = half_wave_sum(o);
    if (lane32 == 0) {
      put<BF16>(O, tk * d_v + r, o);
      U[tk * d_v + r] = u;
    }
  }
}

// slot[b] <- the accepted node's state, per head (accept -1: unchanged)
__global__ __launch_bounds__(kThreads) void snapshot_commit_kernel(
    const float* __restrict__ snap, float* __restrict__ state_pool, const int32_t* __restrict__ slot,
    const int32_t* __restrict__ tree_off, const int32_t* __restrict__ accept, int32_t H,
    int64_t sz4) {
  const int b = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int a = accept[b];
  if (a < 0) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(snap) + ((int64_t)(tree_off[b] + a) * H + h) * sz4;
  f32x4* dst = reinterpret_cast<f32x4*>(state_pool) + ((int64_t)slot[b] * H + h) * sz4;
  for (int64_t i = threadIdx.x; i < sz4; i += kThreads) dst[i] = src[i];
}

}  // namespace

#define BASELINE_API extern "C" __attribute__((visibility("default")))

// One tree depth of one layer: n_level (node, head) pairs, nodes listed in
// level_nodes.  parent_node[N] holds each node's parent as a global node index
// (-1 for a root), node_tree[N] its tree.  Returns 0, or 2 for a bad size and
// 5 for a failed launch.
BASELINE_API int snapshot_level(int32_t bf16, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const float* state_pool,
                                const int32_t* slot, const int32_t* node_tree,
                                const int32_t* parent_node, const int32_t* level_nodes,
                                int32_t n_level, float* snap, void* O, float* U, int32_t H,
                                int32_t d_k, int32_t d_v, void* stream) {
  if (n_level < 1 || H < 1 || d_k < 4 || d_k > 128 * kMaxChunks || d_k % 4 || d_v < 1 ||
      (int64_t)n_level * H >= (1 << 30))
    return 2;
  const dim3 grid(n_level * H), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(snapshot_level_kernel<true>, grid, block, 0, (hipStream_t)stream, q, k, v,
                       g, beta, state_pool, slot, node_tree, parent_node, level_nodes, snap, O, U,
                       H, d_k, d_v);
  else
    hipLaunchKernelGGL(snapshot_level_kernel<false>, grid, block, 0, (hipStream_t)stream, q, k, v,
                       g, beta, state_pool, slot, node_tree, parent_node, level_nodes, snap, O, U,
                       H, d_k, d_v);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

BASELINE_API int snapshot_commit(const float* snap, float* state_pool, const int32_t* slot,
                                 const int32_t* tree_off, const int32_t* accept, int32_t B,
                                 int32_t H, int32_t d_k, int32_t d_v, void* stream) {
  if (B < 1 || H < 1 || (d_k * d_v) % 4 || (int64_t)B * H >= (1 << 30)) return 2;
  hipLaunchKernelGGL(snapshot_commit_kernel, dim3(B * H), dim3(kThreads), 0, (hipStream_t)stream,
                     snap, state_pool, slot, tree_off, accept, H, (int64_t)d_k * d_v / 4);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
