// Tile geometry and fragment helpers shared by the verify kernels of libbole.
#pragma once

#include <type_traits>

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

// The previous round's accepted path, committed into the slot by the verify
// kernel before it reads the state (bole_commit_tree_verify).  Request b of the
// round is request b of the previous round, with the same slot.
struct CommitIO {
  float* pool;              // [n_slots, H, d_v, d_k] state pool, updated in place
  const void* k;            // [N0, H, d_k] the previous round's keys (token dtype)
  const float* U;           // [N0, H, d_v] the previous round's U
  const float* logP;        // [N0, H] the previous round's gate sums
  const uint64_t* anc;      // [N0] ancestor-or-self sets of the previous forest
  const int32_t* tree_off;  // [B + 1] the previous forest's offsets
  const int32_t* accept;    // [B] accepted local node, -1 for nothing to commit
  int32_t N;                // N0
};

// The n-th (from 0) set bit of m, by binary search over halves.  If m has n
// or fewer set bits the result is some position in 0..63.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  int pos = 0;
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const uint64_t low = m & ((1ull << half) - 1ull);
    const int c = __popcll(low);
    const bool up = n >= c;
    n -= up ? c : 0;
    m = up ? m >> half : low;
    pos += up ? half : 0;
  }
  return pos;
}

// The accepted-path update S <- P_a S + sum_j (P_a / P_j) U_j k_j^T on the state
// rows one verify lane holds: value column v, keys 32 kk + 8 g .. + 7 for each
// 32-key chunk kk.  It takes the MFMA steps of bole_commit_path on the same
// operands, so both produce the same bits.  Each 8-key group is two 16x16
// accumulator tiles whose row m is key 32 kk + 8 (m / 4) + 4 half + m % 4, so a
// lane's accumulator holds exactly its four keys of the group: the update needs
// no data movement between lanes.  The A operand (keys) of a lane is row m =
// l16 of that tile at its four path positions, the B operand (P_a/P_j) U_j[v]
// at the same positions, split hi + lo.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte store at a uniform base address plus a 32-bit byte offset per lane
// (the compiler keeps the base in scalar registers).
__device__ __forceinline__ void store_at(float* base, uint32_t off_bytes, const f32x4& v) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + off_bytes) = v;
}

// Wait states before a cross-lane read-out, from the CDNA4 (gfx950) table of
// required independent instructions (the hazards the hardware does not
// interlock), kept in place by scheduling barriers:
//  - an XDL (MFMA) VGPR result read by a VALU instruction: passes + 4 on
//    gfx950; v_mfma_f32_16x16x16_bf16 takes 4 passes, so 8 (s_nop 7);
//  - a VALU VGPR write read by v_permlane16_swap / v_permlane32_swap (either
//    operand: both are read and written) or by a DPP instruction: 2 (s_nop 1).
// The compiler's own hazard pass for gfx950 inserts the same counts (s_nop 7
// after such an MFMA, s_nop 1 before a swap or a DPP read of a fresh VALU
// result); the explicit waits hold them at the stage boundaries whatever the
// scheduler interleaves.
__device__ __forceinline__ void xdl_read_gap() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void cross_lane_gap() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

template <int DT>
struct PathCommit {
  using KRaw = std::conditional_t<DT == BOLE_BF16, uint16_t, uint32_t>;
  using KVec = std::conditional_t<DT == BOLE_BF16, u16x4, u32x4>;
  static constexpr int NK = StageCfg<DT>::KC / 32;  // 32-key chunks per lane
  const KRaw* kp;   // keys of head h at node 0 of the previous tree
  const float* up;  // U of head h at node 0 (uniform; the lane adds its column)
  int64_t kstr, ustr;
  int ucol;         // the lane's value column (clamped into the row)
  uint64_t path;
  float lp, lpa, Pa;
  int La;
  int node[4];      // the lane's path positions of a step, as node ids
  int kc_;          // the step's first position
  float wt[4];      // P_a / P_j
  float uraw[4];    // U_j[v]

  static __device__ __forceinline__ int key(int kk, int half, int l16) {
    return 32 * kk + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
  }
  // positions kc + 4 g + e of the step: node ids (position 0 past the path)
  __device__ __forceinline__ void nodes(int kc, int g4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = kc + 4 * g4 + e;
      node[e] = nth_set_bit(path, p < La ? p : 0);
    }
    kc_ = kc;
  }
  // bit e: the lane's position e of the step is on the path
  __device__ __forceinline__ uint32_t lmask(int g4) const {
    const int left = La - kc_ - 4 * g4;
    return left >= 4 ? 15u : (left > 0 ? (1u << left) - 1u : 0u);
  }
  // their U loads (unconditional)
  __device__ __forceinline__ void load_u() {
#pragma unroll
    for (int e = 0; e < 4; ++e) uraw[e] = up[(int64_t)node[e] * ustr + ucol];
  }
  // and their weights P_a / P_j
  __device__ __forceinline__ void weights() {
#pragma unroll
    for (int e = 0; e < 4; ++e) wt[e] = expf(lpa - __shfl(lp, node[e]));
  }
  // the step's B fragments: (P_a/P_j) U_j[v], split hi + lo
  __device__ __forceinline__ void bfrag(bool vin, int g4, bf16x4& bh, bf16x4& bl) const {
    const uint32_t lm = lmask(g4);
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, wt[e] * uraw[e]) &
                                           keep(vin && ((lm >> e) & 1u)));
    split_bf16x4(x, bh, bl);
  }
  // A step's key rows are staged once per workgroup, transposed: row c holds
  // key c of the 16 path positions, so a lane's A fragment (four consecutive
  // positions of one key) is one LDS read.  The four 4-position groups of row
  // c are XOR-swizzled by (c / 8) % 4: the keys a read instruction touches in
  // one 16-lane group then fall in distinct banks.  Thread t loads 8 bytes of
  // position kc + t / 32 (unconditionally, a key past d_k reads key 0) and
  // writes them once they land.
  static constexpr int KPT = 8 / sizeof(KRaw);  // keys per thread
  using KPiece = std::conditional_t<DT == BOLE_BF16, u16x4, uint2>;
  __device__ __forceinline__ KPiece tile_load(int t, int kc, int d_k) const {
    const int p = kc + (t >> 5), c = KPT * (t & 31);
    const int n = nth_set_bit(path, p < La ? p : 0);
    return *reinterpret_cast<const KPiece*>(kp + (int64_t)n * kstr + (c < d_k ? c : 0));
  }
  static __device__ __forceinline__ int tile_at(int c, int p) {
    return c * 16 + (p ^ (((c >> 3) & 3) << 2));
  }
  __device__ __forceinline__ void tile_store(KRaw* kt, int t, const KPiece& v) const {
    const int p = t >> 5, c = KPT * (t & 31);
#pragma unroll
    for (int i = 0; i < KPT; ++i) kt[tile_at(c + i, p)] = v[i];
  }
  // the whole tile for step kc, by every thread of the workgroup (uniform)
  __device__ __forceinline__ void stage(KRaw* kt, int kc, int d_k) const {
    const KPiece v = tile_load(threadIdx.x, kc, d_k);
    __syncthreads();  // the previous step's tile is no longer read
    tile_store(kt, threadIdx.x, v);
    __syncthreads();
  }

  // one step of 16 path positions onto chunks [k0, k1) of the lane's rows; the
  // first starts the accumulation from P_a S.  Keys from the staged tile.
  __device__ __forceinline__ void apply(float (&sx)[NK][8], int k0, int k1, bool first,
                                        const bf16x4& bh, const bf16x4& bl, int l16, int g4, int d_k,
                                        const KRaw* kt) const {
    const uint32_t lm = lmask(g4);
#pragma unroll
    for (int kk = k0; kk < k1; ++kk)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = key(kk, half, l16);
        const uint32_t kok = keep(c < d_k);
        const KVec kv = *reinterpret_cast<const KVec*>(kt + tile_at(c, 4 * g4));
        bf16x4 ah, al;
        if (DT == BOLE_BF16) {
          u16x4 raw;
#pragma unroll
          for (int e = 0; e < 4; ++e) raw[e] = kv[e] & (uint16_t)(keep((lm >> e) & 1u) & kok);
          ah = __builtin_bit_cast(bf16x4, raw);
        } else {
          f32x4 kx;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            kx[e] = __builtin_bit_cast(float, kv[e] & (keep((lm >> e) & 1u) & kok));
          split_bf16x4(kx, ah, al);
        }
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = first ? Pa * sx[kk][4 * half + i] : sx[kk][4 * half + i];
        acc = mfma16_bf16(ah, bh, acc);
        acc = mfma16_bf16(ah, bl, acc);
        if (DT == BOLE_F32) acc = mfma16_bf16(al, bh, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[kk][4 * half + i] = acc[i];
      }
  }
  // the steps from position kc0 on, on every chunk, each with its own staged
  // tile (uniform over the workgroup: it has barriers)
  __device__ __forceinline__ void steps(float (&sx)[NK][8], KRaw* kt, int kc0, bool vin, int g4,
                                        int l16, int d_k) {
    for (int kc = kc0; kc < La; kc += 16) {
      stage(kt, kc, d_k);
      nodes(kc, g4);
      load_u();
      weights();
      bf16x4 bh, bl;
      bfrag(vin, g4, bh, bl);
      apply(sx, 0, NK, kc == 0, bh, bl, l16, g4, d_k, kt);
    }
  }
  // Committed chunks [k0, k1) back into the slot, as whole 128-byte lines (the
  // state rows leave in the middle of the kernel, so ordinary write-back stores
  // measured faster than writing through: 24.5 against 26.0 us at the target
  // shape; 16-byte pieces at a 32-byte stride, written through, took 31.9).  A
  // chunk of row v
  // is one line, held as 32 bytes by each of the four lanes g = 0..3 of column
  // v.  Two row swaps between the lane's halves (16-lane rows, then 32-lane
  // halves) leave each lane with the line's 16-byte pieces g (first half) and
  // 4 + g (second half); a rotation by 8 within each 16-lane row then lets one
  // store cover rows 0..7 of the wave's 16 and the next rows 8..15, each line
  // whole.  base is the wave's first row (uniform).
  __device__ __forceinline__ void store(float* base, const float (&sx)[NK][8], int k0, int k1,
                                        int v_left, int l16, int g4, int d_k) const {
    const bool low = l16 < 8;
    const int row1 = l16 & 7, row2 = row1 + 8;
    const int c_half = (low ? 0 : 16) + 4 * g4;  // the lane's key within a chunk
#pragma unroll
    for (int kk = k0; kk < k1; ++kk) {
      // The update's accumulators are MFMA results, read out by the swaps'
      // operand copies (8 wait states); each swap stage and the rotation read
      // the previous stage's VALU writes (2 each).
      uint32_t x0[4], x1[4];
      xdl_read_gap();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, sx[kk][i]),
                                                          __builtin_bit_cast(uint32_t, sx[kk][4 + i]),
                                                          false, false);
        x0[i] = s16[0];
        x1[i] = s16[1];
      }
      cross_lane_gap();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto s32 = __builtin_amdgcn_permlane32_swap(x0[i], x1[i], false, false);
        x0[i] = s32[0];  // line piece g4 (keys 4 g4 .. + 3)
        x1[i] = s32[1];  // line piece 4 + g4
      }
      cross_lane_gap();
      f32x4 d1, d2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // both halves rotate by 8 within the 16-lane row and the select comes
        // after the move (a select on the rotated operand was folded away by
        // the compiler, which is wrong for a cross-lane move)
        const int r0 = __builtin_amdgcn_update_dpp(0, (int)x0[i], 0x128, 0xf, 0xf, false);
        const int r1 = __builtin_amdgcn_update_dpp(0, (int)x1[i], 0x128, 0xf, 0xf, false);
        d1[i] = __builtin_bit_cast(float, low ? (int)x0[i] : r1);
        d2[i] = __builtin_bit_cast(float, low ? r0 : (int)x1[i]);
      }
      const int c = 32 * kk + c_half;
      if (c - 4 * g4 < d_k) {  // the 16-key half is inside d_k (d_k is a multiple of 16)
        if (row1 < v_left) store_at(base, 4u * (uint32_t)(row1 * d_k + c), d1);
        if (row2 < v_left) store_at(base, 4u * (uint32_t)(row2 * d_k + c), d2);
      }
    }
  }
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
