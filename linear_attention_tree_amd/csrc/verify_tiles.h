// Tile geometry and fragment helpers shared by the verify kernels of libbole.
#pragma once

#include "common.h"

namespace bole {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBV = 16 * kWaves;  // value columns per workgroup

template <int DT>
struct StageCfg {
  static constexpr int KC = DT == BOLE_BF16 ? 128 : 64;  // d_k chunk staged per pass
  static constexpr int LROW = KC;                         // bf16 per LDS row
  static constexpr int CHUNKS = KC / 8;                   // 16-byte chunks per row
  static constexpr int NMAT = DT == BOLE_BF16 ? 2 : 4;    // Q, K (hi) [+ Q, K lo]
};

// XOR swizzle of 16-byte chunks within a staged row: the 16 rows an A fragment
// reads at one K offset land in 16 different bank groups.
template <int DT>
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ (row & (StageCfg<DT>::CHUNKS - 1));
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

// A [64 rows x kBV columns] tile of the workgroup's value columns in LDS (V on
// the way in, U and O on the way out), row-major with the columns XOR-swizzled
// in blocks of 16 by (row / 4) % 4.  Accumulator-layout accesses (a wave's 16
// columns at rows 4g + e, g = 0..3) then hit four different bank groups, and
// the 4- and 8-element row pieces moved to and from global memory stay
// contiguous.
__device__ __forceinline__ int vtile_idx(int row, int col) {
  return row * kBV + (col ^ (((row >> 2) & 3) << 4));
}

// Tree preparation done inside the verify kernel (bole_tree_verify): its
// inputs and the outputs it publishes for the commit.
struct PrepIO {
  const int32_t* parent;  // [N] local parent, -1 for a root
  const float* g;         // [N, H] log-gates of the layer
  int32_t* depth;         // [N]
  uint64_t* anc;          // [N]
  int32_t* order;         // [N]
  int32_t* tree_depth;    // [B]
  float* logP;            // [N, H] of the layer
};

// How the verify kernel solves (I + G) U = R.  All three are exact (the closed
// form fixes the outputs, not the solve; arXiv page, Theorem 1 discussion).
//  kSolveBlocked  forward substitution over 16-row tiles with the diagonal
//                 blocks' inverses formed while the state streams in
//  kSolveNeumann  the d_b-step propagation Z <- -G Z, U += Z of Eq. 8
//  kSolveInverse  the G and C inputs hold W = (I + G)^-1 and M = C W
constexpr int kSolveBlocked = 0, kSolveNeumann = 1, kSolveInverse = 2;

// Bit flags of the value-tile transfers, set by the host.
// kVecV: d_v is a multiple of the elements in 16 bytes of v and v is 16-byte
// aligned, so V rows move as 16-byte pieces.  kVecOut: d_v % 4 == 0 and U and O
// are aligned for 4-element pieces.
constexpr int kVecV = 1, kVecOut = 2;

template <int DT>
struct VTileCfg {
  static constexpr int EPP = DT == BOLE_BF16 ? 8 : 4;    // elements per 16-byte piece
  static constexpr int PPR = kBV / EPP;                   // pieces per tile row
  static constexpr int PER = kMaxTree * PPR / kThreads;   // pieces per thread
};

// Stage one d_k chunk of the tree's Q and K rows (level order) into LDS as bf16
// (float32 rows are split into hi and lo planes), in two halves: qk_issue puts
// every global load in flight, qk_commit converts and stores them.  Work issued
// between the two overlaps the round trip, and loads issued after qk_issue stay
// in flight while qk_commit waits.
template <int DT>
struct QkCfg {
  static constexpr int EPP = DT == BOLE_BF16 ? 8 : 4;   // elements per 16-byte piece
  static constexpr int PIECES = StageCfg<DT>::KC / EPP;  // pieces per row
  static constexpr int PER = 2 * kMaxTree * PIECES / kThreads;
};

// NODE_ORDER: the rows are fetched in node order (piece row n holds node n), so
// the loads need only the tree's offset; qk_commit then stores node n at its
// level position posOf[n] (positions past the tree keep their index).
template <int DT, bool NODE_ORDER = false>
__device__ __forceinline__ void qk_issue(u16x8* buf, const void* q, const void* k,
                                         const int* rowNode, int T, int off, int H, int h,
                                         int d_k, int kc0) {
  using QC = QkCfg<DT>;
#pragma unroll
  for (int it = 0; it < QC::PER; ++it) {
    const int id = threadIdx.x + kThreads * it;
    const int mat = id / (kMaxTree * QC::PIECES);
    const int rem = id - mat * (kMaxTree * QC::PIECES);
    const int row = rem / QC::PIECES, pc = rem - (rem / QC::PIECES) * QC::PIECES;
    const int kk = kc0 + QC::EPP * pc;
    // unconditional load (row and column clamped into the tree), zeroed after
    const bool in = row < T && kk < d_k;
    const int node = NODE_ORDER ? min(row, T - 1) : rowNode[min(row, T - 1)];
    const int64_t e = ((int64_t)(off + node) * H + h) * d_k + (kk < d_k ? kk : 0);
    const u16x8 val =
        DT == BOLE_BF16
            ? *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(mat == 0 ? q : k) + e)
            : *reinterpret_cast<const u16x8*>(reinterpret_cast<const float*>(mat == 0 ? q : k) + e);
    const u16x8 zero = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    buf[it] = in ? val : zero;  // a select of a loaded value: the load stays unconditional
  }
}

template <int DT, bool NODE_ORDER = false>
__device__ __forceinline__ void qk_commit(__bf16* stage, const u16x8* buf,
                                          const int* posOf = nullptr, int T = 0) {
  using SC = StageCfg<DT>;
  using QC = QkCfg<DT>;
#pragma unroll
  for (int it = 0; it < QC::PER; ++it) {
    const int id = threadIdx.x + kThreads * it;
    const int mat = id / (kMaxTree * QC::PIECES);
    const int rem = id - mat * (kMaxTree * QC::PIECES);
    const int r0 = rem / QC::PIECES, pc = rem - (rem / QC::PIECES) * QC::PIECES;
    const int row = NODE_ORDER && r0 < T ? posOf[r0] & (kMaxTree - 1) : r0;
    if (DT == BOLE_BF16) {
      *reinterpret_cast<u16x8*>(stage + (mat * kMaxTree + row) * SC::LROW + 8 * swz<DT>(row, pc)) =
          buf[it];
    } else {
      const f32x4 x = __builtin_bit_cast(f32x4, buf[it]);
      bf16x4 hi, lo;
      split_bf16x4(x, hi, lo);
      // 4 elements = half a 16-byte chunk
      const int ch = swz<DT>(row, pc >> 1), half = pc & 1;
      *reinterpret_cast<bf16x4*>(stage + (mat * kMaxTree + row) * SC::LROW + 8 * ch + 4 * half) = hi;
      *reinterpret_cast<bf16x4*>(stage + ((2 + mat) * kMaxTree + row) * SC::LROW + 8 * ch +
                                 4 * half) = lo;
    }
  }
}

// G and C are parked in LDS already split into bf16 hi/lo planes (G negated),
// each plane 64 rows x 64 entries, laid out for the A fragments of
// v_mfma_f32_16x16x32_bf16 with a permuted K order: the 32 K positions of block
// (I, J) cover the two 16-row tiles 2J and 2J+1, and lane l's eight positions
// 8*(l/16) + e map to row 4*(l/16) + (e & 3) of tile 2J + (e >> 2).  With that
// order a lane's B fragment is just its own accumulator entries of tiles 2J and
// 2J+1 (16x16 accumulator layout: rows 4*(l/16) .. +3 of column l%16), so the
// recursion never moves Z or U between lanes.  Within a row, the 16-byte chunk
// (J, l/16) holding a fragment is XOR-swizzled so 16 rows hit distinct banks.
// Blocks: (I, J) with J <= I/2, index kBlk(I, J) in {0..5}.
constexpr int kGcPlane = kMaxTree * kMaxTree;  // bf16 per plane

__device__ __forceinline__ int gc_pos(int row, int col) {
  const int J = col >> 5, c32 = col & 31;
  const int chunk = (J << 2) | ((c32 & 15) >> 2);
  const int phys = chunk ^ ((row >> 1) & 7);
  return row * kMaxTree + phys * 8 + ((c32 >> 4) << 2) + (c32 & 3);
}

__device__ __forceinline__ int gc_frag(int row, int J, int g) {
  return row * kMaxTree + (((J << 2) | g) ^ ((row >> 1) & 7)) * 8;
}

__device__ __forceinline__ constexpr int kBlk(int I, int J) { return I < 2 ? I : 2 + 2 * (I - 2) + J; }

__device__ __forceinline__ void load_tri_blocks(const __bf16* hi_plane, const __bf16* lo_plane,
                                                int nmt, int lane, bf16x8* hi, bf16x8* lo) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int J = 0; J <= I / 2; ++J) {
      const int idx = kBlk(I, J);
      if (I < nmt) {
        const int o = gc_frag(16 * I + l16, J, g);
        hi[idx] = *reinterpret_cast<const bf16x8*>(hi_plane + o);
        lo[idx] = *reinterpret_cast<const bf16x8*>(lo_plane + o);
      } else {
        hi[idx] = zero_bf16x8();
        lo[idx] = zero_bf16x8();
      }
    }
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& a, const f32x4& b) {
  const f32x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ void split_pair(const f32x4& a, const f32x4& b, bf16x8& hi,
                                           bf16x8& lo) {
  const f32x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  hi = __builtin_convertvector(v, bf16x8);
  lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x8), bf16x8);
}

// The ten lower-triangle tiles (I >= J) of a 64x64 Gram product, computed in
// the fused variant: the four diagonal tiles first.
__constant__ constexpr int kTileI[10] = {0, 1, 2, 3, 1, 2, 2, 3, 3, 3};
__constant__ constexpr int kTileJ[10] = {0, 1, 2, 3, 0, 0, 1, 0, 1, 2};

}  // namespace bole
