// Value-tiled closed-form verification (Bole, arXiv page section IV-B; the
// review's Theorem 1 and Eqs. 6-8).  One workgroup per (tree b, head h, value
// tile r) of kBV value columns; the tree is never split across workgroups.  At
// d_v = 128 a head is one workgroup and the whole forest fits on the chip in a
// single round.
//
// Rows are taken in level order (nodes sorted by depth, the order produced by
// tree preparation).  That is a parent-before-child indexing, so G is strictly
// lower triangular and C lower triangular (arXiv page, Theorem 1 discussion).
//
// The structured system (I + G) U = R is solved by forward substitution over
// the four 16-row tiles, which the pages allow (the closed form fixes the
// outputs, not how the system is solved).  Each diagonal block's inverse is the
// finite Neumann series of Eq. 8 restricted to the tile; it depends on Q, K,
// beta and the gates only, so it is formed while the state slice is in flight.
//
//  Gram     (fused variant) Q K^T and K K^T from the staged rows, masked
//           epilogue, into bf16 hi/lo planes of -G and C in LDS.
//  Diag     waves 0-3: (I + G_tt)^-1 for tile t by repeated squaring.
//  Phase A  [Q;K] S_pre^(r) on v_mfma_f32_16x16x32_bf16: Q/K rows staged once
//           in LDS (level order), S_pre rows of the wave's 16 value columns
//           loaded straight into B fragments and split into bf16 hi+lo
//           (float32 Q/K split too).  B0 = D_P QS, R = D_beta (V - D_P KS).
//  Solve    U_t = (I + G_tt)^-1 (R_t - sum_{s<t} G_ts U_s), tile by tile, with
//           a permuted K order (load_tri_blocks) that makes the lane's own U
//           tiles the B operand: U never leaves registers.
//  Readout  O = B0 + C U, float32 accumulation.  Every product splits its
//           float32 operands hi + lo, O's own (Q S_pre, C U) included.
//  Stores   U (compact, float32) and O (token dtype) pass through LDS tiles and
//           leave as 4-element pieces of the nodes' rows; V arrives the same
//           way, as 16-byte row pieces staged for the accumulator layout.
//
// COMMIT (bole_commit_tree_verify): before phase A reads the state, the
// previous round's accepted path is committed into it (paper Eq. 10) in the
// lane's registers, with bole_commit_path's MFMA steps on the same operands
// (PathCommit), and the committed rows are written back to the slot; the
// verify then uses them as S_pre.
//
// Two other exact solves can be selected (SOLVE):
//  Neumann  the d_b-step propagation of Eq. 8 as the pages run it: Z <- -G Z,
//           U += Z, starting from Z = U = R.  Z^(m) = (-G)^m R vanishes on rows
//           shallower than m, so a step skips row tiles whose deepest row is
//           above m and input tiles whose deepest row is above m - 1.
//  Inverse  the G and C inputs hold W = (I + G)^-1 and M = C W (formed by
//           bole_factor_inverse): U = W R and O = B0 + M R, two independent
//           products with no chain between tiles.
#include <algorithm>
#include <type_traits>

#include "tree_topo.h"
#include "verify_tiles.h"

namespace bole {

// FUSED = false: G and C come from bole_factor_gc.  FUSED = true: the Gram
// products and their masked epilogue run here, from the Q/K rows already staged
// for the state contractions, with the same arithmetic as bole_factor_gc (d_k
// must fit one staged chunk).  ONE: d_k fits one staged chunk (always so when
// fused), which drops the re-staging loop and its registers.  PREP (fused only):
// the kernel derives the tree's topology and this head's gate sums itself from
// the parents and log-gates, with the arithmetic of bole_tree_prep, and
// publishes them for the commit; the order/depth/anc/logP inputs are unused.
// COMMIT (with PREP): the previous round's accepted path of this layer is
// committed into the slot first (CommitIO), and the verify reads the updated
// state from registers.
// EARLY (bf16 tokens, blocked solve, V readable as 8-byte pieces): the solve's
// operands are made visible before phase A and V reaches the accumulator layout
// through one MFMA against the identity instead of an LDS tile, so each wave
// goes from its phase A to its solve and readout without waiting for the
// others.
template <int DT, bool FUSED, bool ONE, bool PREP, int SOLVE = kSolveBlocked, bool COMMIT = false,
          bool EARLY = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void verify_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ logP, const float* __restrict__ beta,
    const float* __restrict__ state_pool, int32_t n_slots, const int32_t* __restrict__ slot,
    const float* __restrict__ G, const float* __restrict__ C, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ order,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ tree_off,
    const int32_t* __restrict__ tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
    int32_t d_v, void* __restrict__ O, float* __restrict__ U, int32_t vecf, PrepIO prep,
    uint32_t* __restrict__ err, CommitIO cm) {
  using SC = StageCfg<DT>;
  static_assert(!(FUSED && SOLVE == kSolveInverse), "W and M come from bole_factor_inverse");
  static_assert(!COMMIT || (FUSED && PREP && SOLVE == kSolveBlocked), "commit inside tree verify");
  static_assert(!EARLY || (DT == BOLE_BF16 && SOLVE == kSolveBlocked), "early tail: bf16, blocked");
  __shared__ __align__(16) __bf16 stage[SC::NMAT * kMaxTree * SC::LROW];
  // planes: -G hi, -G lo, C hi, C lo
  __shared__ __align__(16) __bf16 gcs[4 * kGcPlane];
  __shared__ __align__(16) float rowP[kMaxTree], rowBeta[kMaxTree], rowE2[kMaxTree];
  __shared__ uint64_t rowApos[kMaxTree];  // ancestor-or-self set in level positions
  __shared__ int posOf[kMaxTree];         // local node id -> level position
  __shared__ int rowDep[kMaxTree];
  __shared__ __align__(16) int rowNode[kMaxTree];
  __shared__ bf16x4 invs[4][2][64];  // (I + G_tt)^-1, A layout, hi / lo
  __shared__ int tree_ok;
  // COMMIT: the first path step's key rows, transposed (key, position)
  __shared__ __align__(16) typename PathCommit<DT>::KRaw ktile[COMMIT ? 16 * SC::KC : 1];

  const int NV = (d_v + kBV - 1) / kBV;
  const int lid = xcd_remap(blockIdx.x, B * H * NV);
  const int unit = lid / NV, r = lid - (lid / NV) * NV;
  const int b = unit / H, h = unit - (unit / H) * H;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform
  const int g4 = lane >> 4, l16 = lane & 15;

  // independent per-tree scalars, fetched together
  const int off_in = tree_off[b], end_in = tree_off[b + 1];
  const int td = PREP ? 0 : tree_depth[b];
  const int s = slot[b];
  const bool range_bad =
      off_in < 0 || end_in > N || end_in - off_in < 1 || end_in - off_in > kMaxTree;
  // COMMIT: a workgroup whose tree range is bad still commits.  It runs on as a
  // stand-in one-node tree at node 0 (every access in bounds) that writes
  // nothing and leaves at the rejected-tree exit.
  const int off = COMMIT && range_bad ? 0 : off_in;
  const int T = COMMIT && range_bad ? 1 : end_in - off_in;
  // the previous round's accepted node and tree (COMMIT)
  const int pa = COMMIT ? cm.accept[b] : -1;
  const int po = COMMIT ? cm.tree_off[b] : 0;
  const int pT = COMMIT ? cm.tree_off[b + 1] - po : 1;
  const bool reporter = threadIdx.x == 0 && h == 0 && r == 0;
  const bool slot_ok = s >= 0 && s < n_slots;
  bool pend = false;  // uniform: a path to commit into the slot
  if (COMMIT && pa != -1 && slot_ok) {
    if (po < 0 || pT < 1 || pT > kMaxTree || po > cm.N - pT) {
      if (reporter) report(err, BOLE_ERR_TREE_SIZE);
    } else if (pa < 0 || pa >= pT) {
      if (reporter) report(err, BOLE_ERR_BAD_ACCEPT);
    } else {
      pend = true;
    }
  }

  // The state rows this lane holds: value column vcol of the slot, keys
  // 32 kk + 8 g4 .. + 7 (the B fragments of phase A).
  const int vloc = 16 * w + l16;
  const int vcol = kBV * r + vloc;
  const bool vin = vcol < d_v;
  const int64_t srow = (((int64_t)(COMMIT && !slot_ok ? 0 : s) * H + h) * d_v + (vin ? vcol : 0)) * d_k;
  const float* Srow = state_pool + srow;
  // COMMIT: the wave's first slot row (uniform), where the committed rows go
  float* const cbase =
      cm.pool + (((int64_t)(slot_ok ? s : 0) * H + h) * d_v + kBV * r + 16 * w) * d_k;
  const int cvl = d_v - (kBV * r + 16 * w);  // rows of the wave inside d_v
  float sx[SC::KC / 32][8];
  // K positions past d_k read the row's first entries instead: they meet staged
  // Q/K columns that are zero.  Lanes past d_v compute columns never stored.
  auto load_s = [&](int kc0, int k0, int k1) {
#pragma unroll
    for (int kk = k0; kk < k1; ++kk) {
      const int kidx = kc0 + 32 * kk + 8 * g4;
      load_f32x8(Srow + (kidx < d_k ? kidx : 0), sx[kk]);
    }
  };

  // COMMIT: the path (the accepted node's ancestor-or-self set) and the gate
  // sums of the previous tree, one node per lane; loads clamped to node 0 when
  // nothing is to be committed
  PathCommit<DT> pc;
  if (COMMIT) {
    const int a0 = pend ? pa : 0, o0 = pend ? po : 0, t0 = pend ? pT : 1;
    // the set is cut to the tree's nodes and never empty (an empty one, which
    // only bad data can give, becomes the node itself), so every path position
    // below La names a node of the previous tree
    const uint64_t pm = cm.anc[o0 + a0] & (t0 == 64 ? ~0ull : ((1ull << t0) - 1ull));
    const uint64_t pth = pm ? pm : 1ull << a0;
    // uniform (one load address for the whole workgroup), held in scalar
    // registers so that branches on the path length are scalar branches
    pc.path = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(pth >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pth);
    pc.lp = cm.logP[(int64_t)(o0 + min(lane, t0 - 1)) * H + h];
    pc.kp = reinterpret_cast<const typename PathCommit<DT>::KRaw*>(cm.k) + (int64_t)o0 * H * d_k +
            (int64_t)h * d_k;
    pc.up = cm.U + (int64_t)o0 * H * d_v + (int64_t)h * d_v;
    pc.ucol = vin ? vcol : 0;
    pc.kstr = (int64_t)H * d_k;
    pc.ustr = (int64_t)H * d_v;
    pc.La = __popcll(pc.path);
  }
  // the whole commit of the lane's rows, for a workgroup that verifies nothing
  constexpr int kNK = SC::KC / 32;
  auto commit_only = [&]() {
    load_s(0, 0, kNK);
    pc.lpa = __shfl(pc.lp, pa);
    pc.Pa = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, expf(pc.lpa))));
    pc.steps(sx, ktile, 0, vin, g4, l16, d_k);
    pc.store(cbase, sx, 0, kNK, cvl, l16, g4, d_k);
  };

  if (range_bad) {
    if (reporter) report(err, BOLE_ERR_TREE_SIZE);
    if (!(COMMIT && pend)) return;
  }
  if (td < 0) return;  // rejected by tree preparation
  if (!slot_ok) {
    if (reporter) report(err, BOLE_ERR_BAD_SLOT);
    return;
  }
  const int nmt = (T + 15) >> 4;

  // Every global load below is unconditional (indices are clamped into the
  // tree and values masked afterwards): a load behind a divergent branch makes
  // the wait for it conservative, and it would then wait for every load issued
  // after it as well.
  // level-order rows: row p holds node order[p].  With PREP wave 0 fetches
  // what the topology and the row tables are built from instead.
  const int nl = off + min(lane, T - 1);
  const int ord = PREP ? 0 : order[nl];
  int p_raw = -1;
  float g_raw = 0.0f, bt_raw = 0.0f;
  if (PREP && w == 0) {  // uniform
    p_raw = prep.parent[nl];
    g_raw = prep.g[(int64_t)nl * H + h];
    bt_raw = beta[(int64_t)nl * H + h];
  }
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

  const int node_l = lane < T ? clamp_node(ord, T) : 0;
  u16x8 qkbuf[QkCfg<DT>::PER];
  typename PathCommit<DT>::KPiece kpiece;
  if (PREP) {
    // the Q/K rows go out now, in node order, behind wave 0's small loads;
    // the topology is derived while they stream in
    qk_issue<DT, true>(qkbuf, q, k, nullptr, T, off, H, h, d_k, 0);
    // COMMIT: the path's key rows and the lane's U entries of its first 16
    // positions, right behind them (they need only the path set, which came
    // with the first scalar loads)
    if (COMMIT) {
      kpiece = pc.tile_load(threadIdx.x, 0, d_k);
      pc.nodes(0, g4);
      pc.load_u();
    }
    __builtin_amdgcn_sched_barrier(0);
    if (w == 0) {
      // tree preparation for this (tree, head): topology (tree_topo.h), then
      // logP level by level, logP_i = logP_parent(i) + g_i from +0 at the roots:
      // the float32 adds of bole_tree_prep's root-first running sum, in order
      const TreeTopo tp = tree_topology(lane, T, p_raw);
      const bool row_in = lane < T;
      if (!tp.fail && !(COMMIT && range_bad)) {
        // the ancestor-or-self set in level positions follows the same
        // recursion, apos_i = apos_parent(i) | bit(pos_i), in the same rounds
        const int pos = tp.pos;
        const int src = max(p_raw, 0);
        float lp = 0.0f;
        uint64_t apos = 0ull;
        for (int lev = 0; lev <= tp.dmax; ++lev) {
          const float lpp = __shfl(lp, src);
          const uint64_t app = __shfl(apos, src);
          if (tp.dep == lev) {
            lp = __fadd_rn(lev == 0 ? 0.0f : lpp, g_raw);
            apos = (lev == 0 ? 0ull : app) | (1ull << pos);
          }
        }
        // row tables at the node's level position (rows past the tree hold
        // node 0 with zero scalars)
        rowNode[pos] = row_in ? lane : 0;
        posOf[lane] = pos;
        const uint32_t rk = keep(row_in);
        rowP[pos] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, expf(lp)) & rk);
        rowBeta[pos] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, bt_raw) & rk);
        rowE2[pos] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, lp * kLog2e) & rk);
        rowDep[pos] = row_in ? tp.dep : 0x7fff;
        rowApos[pos] = apos;  // zero past the tree
        if (row_in && r == 0) {
          prep.logP[(int64_t)(off + lane) * H + h] = lp;
          if (h == 0) {
            prep.depth[off + lane] = tp.dep;
            prep.anc[off + lane] = tp.anc;
            prep.order[off + pos] = lane;
          }
        }
      }
      if (lane == 0) {
        tree_ok = !tp.fail && !(COMMIT && range_bad);
        if (h == 0 && r == 0 && !(COMMIT && range_bad)) {
          prep.tree_depth[b] = tp.fail ? -1 : tp.dmax;
          if (tp.fail) report(err, tp.fail);
        }
      }
    }
  } else if (threadIdx.x < kMaxTree) {
    rowNode[threadIdx.x] = node_l;
    if (lane < T) posOf[node_l] = lane;
  }
  __syncthreads();  // rowNode visible (and with PREP every row table)
  if (PREP && !tree_ok) {  // uniform: a rejected tree
    if (COMMIT && pend) commit_only();
    return;
  }
  if (COMMIT) {
    // the weights of the lane's first 16 path positions (their U entries and
    // key rows are in flight since the Q/K rows)
    pc.lpa = __shfl(pc.lp, pend ? pa : 0);
    pc.Pa = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, expf(pc.lpa))));
    pc.weights();
  }

  // everything below depends on the rows only.  Issue order: the Q/K rows
  // (needed first), the row scalars (wave 0), then the state slice and V,
  // which are consumed last.
  if (!PREP) qk_issue<DT>(qkbuf, q, k, rowNode, T, off, H, h, d_k, 0);

  // nothing that waits on a load may be scheduled above this point: the Q/K
  // rows are in flight before the first wait
  __builtin_amdgcn_sched_barrier(0);

  // park G (negated) and C in LDS, split once into bf16 hi/lo planes
#pragma unroll
  for (int it = 0; it < (FUSED ? 0 : kGcPer); ++it) {
    const int id = threadIdx.x + kThreads * it;
    const int mat = id >> 10, rem = id & 1023;
    const int row = rem >> 4, c4 = rem & 15;
    bf16x4 hi, lo;
    // the substitution and the propagation use -G; the inverse solve W as is
    split_bf16x4(mat || SOLVE == kSolveInverse ? gcr[it] : -gcr[it], hi, lo);
    const int o = gc_pos(row, 4 * c4);
    *reinterpret_cast<bf16x4*>(gcs + (2 * mat) * kGcPlane + o) = hi;
    *reinterpret_cast<bf16x4*>(gcs + (2 * mat + 1) * kGcPlane + o) = lo;
  }
  if (!PREP && w == 0) {
    // The row tables are built by one wave: each row-scalar load touches 64
    // different cache lines (the rows are H elements apart), so eight copies
    // would crowd the address units while the Q/K rows stream in.  Rows past
    // the tree are cleared by masks, not selects (no branch for the loads to
    // sink into).
    const int64_t tok_l = (int64_t)(off + node_l) * H + h;
    const int dep_raw = depth[off + node_l];
    const float lp_raw = logP[tok_l];
    const float bt_raw = beta[tok_l];
    const uint64_t an_raw = FUSED ? anc[off + node_l] : 0ull;
    const bool row_in = lane < T;
    const uint32_t rk = keep(row_in);
    rowP[lane] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, expf(lp_raw)) & rk);
    rowBeta[lane] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, bt_raw) & rk);
    rowE2[lane] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, lp_raw * kLog2e) & rk);
    if (FUSED) {
      // the row's ancestor mask moved from node ids to level positions, where
      // four consecutive columns are four consecutive bits
      uint64_t m = an_raw & (T == 64 ? ~0ull : ((1ull << T) - 1ull)), apos = 0ull;
      while (m) {
        apos |= 1ull << posOf[__builtin_ctzll(m)];
        m &= m - 1ull;
      }
      rowApos[lane] = apos & (0ull - (uint64_t)row_in);
    }
    // depth of level-order row `lane` (nondecreasing in the row index)
    rowDep[lane] = row_in ? dep_raw : 0x7fff;
  }
  if (PREP)
    qk_commit<DT, true>(stage, qkbuf, posOf, T);  // waits for the Q/K rows
  else
    qk_commit<DT>(stage, qkbuf);
  if (COMMIT) pc.tile_store(ktile, threadIdx.x, kpiece);
  __syncthreads();  // staged rows and row tables visible
  // The state slice and V are requested only once the workgroup's Q/K rows are
  // in: the memory system serves concurrent requests interleaved, so issued
  // together (or while sibling waves still wait for their rows) they would
  // delay the Q/K rows, needed first for the Gram products and the diagonal
  // blocks, to the end of the whole transfer; issued after them they still
  // complete as early.  Issuing the slice stalls each wave while the address
  // unit works through it, so the fused variant issues half of it before its
  // first Gram tile and half after, where the stall overlaps Gram work.
  constexpr int kSChunks = SC::KC / 32, kSHalf = SC::KC / 64;
  load_s(0, 0, FUSED ? kSHalf : kSChunks);
  __builtin_amdgcn_sched_barrier(0);

  if (FUSED) {
    // d_k fits one staged chunk (checked by the host): each Gram tile is
    // finished here, with the operands, accumulation order and masked epilogue
    // of bole_factor_gc, written straight into the split planes.  The product
    // is taken transposed (key rows of tile J as the M operand), so a lane
    // holds row i = 16I + l16 at the four consecutive columns 16J + 4g .. +3:
    // the row's scalars are read once and each plane gets one 8-byte store.
    // Wave w takes lower-triangle tile w (and waves 4, 5 tiles 8, 9) of both
    // products: the K rows of tile J, the mask and the gate ratios are shared
    // by the G and C entries of a tile.  Tiles 0-3 are the diagonal ones, so
    // wave t < 4 produces the block it inverts next and reads back only its
    // own writes: no workgroup barrier follows the Gram, and each wave goes on
    // to its diagonal block or to phase A as soon as its own tiles are done.
    // The planes are next read by other waves in the solve, after the barrier
    // that closes phase A.
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (jb == 1) {
        load_s(0, kSHalf, kSChunks);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int tile = jb == 0 ? w : (w == 4 || w == 5 ? w + 4 : 10);
      if (tile < 10) {
        const int I = kTileI[tile], J = kTileJ[tile];
        if (I < nmt) {
          const int irow = 16 * I + l16, jrow = 16 * J + l16;
          f32x4 accC = zero_f32x4(), accG = zero_f32x4();
#pragma unroll
          for (int kk = 0; kk < SC::KC / 32; ++kk) {
            if (32 * kk < d_k) {
              const int io = irow * SC::LROW + 8 * swz<DT>(irow, 4 * kk + g4);
              const int jo = (kMaxTree + jrow) * SC::LROW + 8 * swz<DT>(jrow, 4 * kk + g4);
              const bf16x8 qi = *reinterpret_cast<const bf16x8*>(stage + io);
              const bf16x8 ki = *reinterpret_cast<const bf16x8*>(stage + kMaxTree * SC::LROW + io);
              const bf16x8 kj = *reinterpret_cast<const bf16x8*>(stage + jo);
              accC = mfma_bf16(kj, qi, accC);
              accG = mfma_bf16(kj, ki, accG);
              if (DT == BOLE_F32) {
                const int lo_off = 2 * kMaxTree * SC::LROW;
                const bf16x8 qil = *reinterpret_cast<const bf16x8*>(stage + lo_off + io);
                const bf16x8 kil =
                    *reinterpret_cast<const bf16x8*>(stage + lo_off + kMaxTree * SC::LROW + io);
                const bf16x8 kjl = *reinterpret_cast<const bf16x8*>(stage + lo_off + jo);
                accC = mfma_bf16(kjl, qi, accC);
                accC = mfma_bf16(kj, qil, accC);
                accG = mfma_bf16(kjl, ki, accG);
                accG = mfma_bf16(kj, kil, accG);
              }
            }
          }
          // branch-free epilogue: every entry is computed and the mask clears
          // the ones outside it (an overflowing ratio there is cleared too)
          const int i = irow, j0 = 16 * J + 4 * g4;
          const uint32_t m4 = (uint32_t)(rowApos[i] >> j0) & 15u;
          const uint32_t d = (uint32_t)(i - j0);
          const uint32_t m4g = m4 & ~(d < 4u ? 1u << d : 0u);  // G has no diagonal
          const float e2i = rowE2[i], bi = rowBeta[i];
          const f32x4 e2j = *reinterpret_cast<const f32x4*>(rowE2 + j0);
          f32x4 vc, vg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ratio = gate_ratio(e2i, e2j[e]);
            const float c = ratio * accC[e];
            const float gneg = -(bi * ratio * accG[e]);
            vc[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c) & keep((m4 >> e) & 1u));
            vg[e] =
                __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, gneg) & keep((m4g >> e) & 1u));
          }
          bf16x4 hi, lo;
          const int o = gc_pos(i, j0);
          split_bf16x4(vg, hi, lo);
          *reinterpret_cast<bf16x4*>(gcs + o) = hi;
          *reinterpret_cast<bf16x4*>(gcs + o + kGcPlane) = lo;
          split_bf16x4(vc, hi, lo);
          *reinterpret_cast<bf16x4*>(gcs + o + 2 * kGcPlane) = hi;
          *reinterpret_cast<bf16x4*>(gcs + o + 3 * kGcPlane) = lo;
        }
      }
    }
  }

  // COMMIT: the first step's B fragments, formed once its U loads are in (they
  // went out before the state slice), so that only the split fragments are
  // held from here on
  bf16x4 cbh, cbl;
  if (COMMIT) pc.bfrag(vin, g4, cbh, cbl);

  // ---------------- Diagonal blocks: (I + G_tt)^-1 per 16-row tile --------
  // In level order G is strictly lower triangular, so each 16x16 diagonal
  // block N = -G_tt is nilpotent and (I + G_tt)^-1 = sum_m N^m, the finite
  // Neumann series of Eq. 8 restricted to the tile.  Its index is at most the
  // number of depths the tile spans (k), and the sum is formed by repeated
  // squaring, W <- W (I + P), P <- P P, starting from W = I + N: after s rounds
  // W covers N^0 .. N^(2^(s+1) - 1).  Wave t < 4 owns tile t.  Everything stays
  // in registers on v_mfma_f32_16x16x16_bf16, whose accumulator layout is its
  // B operand layout: each product X Y is taken twice, as mfma(X_A, Y_B) (the
  // B layout of X Y) and as mfma(Y_B, X_A) (the transpose, i.e. the A layout of
  // X Y), so both operand forms of every factor are at hand.  Operands are
  // split bf16 hi + lo, three products each, float32 accumulation.
  if (SOLVE == kSolveBlocked && w < 4 && w < nmt) {
    const int tb = 16 * w;
    const int k_span = rowDep[min(tb + 15, T - 1)] - rowDep[tb] + 1;
    auto id_entry = [&](int e) { return 4 * g4 + e == l16 ? 1.0f : 0.0f; };
    // N in A layout (row tb + l16, columns tb + 4g .. +3: one 8-byte read) and
    // in B layout (rows tb + 4g .. +3, column tb + l16)
    f32x4 Pa, Pb, Wa, Wb;
    {
      const int oa = gc_pos(tb + l16, tb + 4 * g4);
      const bf16x4 ah = *reinterpret_cast<const bf16x4*>(gcs + oa);
      const bf16x4 al = *reinterpret_cast<const bf16x4*>(gcs + kGcPlane + oa);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ob = gc_pos(tb + 4 * g4 + e, tb + l16);
        Pa[e] = (float)ah[e] + (float)al[e];
        Pb[e] = (float)gcs[ob] + (float)gcs[ob + kGcPlane];
        Wa[e] = Pa[e] + id_entry(e);
        Wb[e] = Pb[e] + id_entry(e);
      }
    }
    auto mm = [&](const f32x4& xa, const f32x4& yb) {  // A-layout x times B-layout y
      bf16x4 xh, xl, yh, yl;
      split_bf16x4(xa, xh, xl);
      split_bf16x4(yb, yh, yl);
      f32x4 acc = mfma16_bf16(xh, yh, zero_f32x4());
      acc = mfma16_bf16(xl, yh, acc);
      return mfma16_bf16(xh, yl, acc);
    };
    for (int span = 2; span < k_span; span *= 2) {
      const f32x4 Pb2 = mm(Pa, Pb), Pa2 = mm(Pb, Pa);  // P P, both layouts
      Pa = Pa2;
      Pb = Pb2;
      f32x4 Qa, Qb;  // I + P
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Qa[e] = Pa[e] + id_entry(e);
        Qb[e] = Pb[e] + id_entry(e);
      }
      const f32x4 Wb2 = mm(Wa, Qb), Wa2 = mm(Qb, Wa);  // W (I + P), both layouts
      Wa = Wa2;
      Wb = Wb2;
    }
    bf16x4 wh, wl;
    split_bf16x4(Wa, wh, wl);
    invs[w][0][lane] = wh;
    invs[w][1][lane] = wl;
  }
  // EARLY: the G/C planes and the diagonal inverses are the only LDS data the
  // solve and readout read that other waves wrote; they are complete here.
  // (The barrier waits for LDS traffic only: the state slice stays in flight.)
  if (EARLY) __syncthreads();

  // ---------------- Phase A: [Q;K] S_pre^(r) ----------------
  // V rows of the workgroup's value columns, requested only now (after the
  // Gram and diagonal work, so they do not compete with it) as 16-byte row
  // pieces, held in registers through phase A and staged through LDS for the
  // accumulator layout afterwards.  Rows past the tree read row T-1 and pieces
  // past d_v column 0; both are zeroed.  Without kVecV every piece reads the
  // aligned block holding v[0] and V is fetched element-wise after phase A.
  // EARLY: the lane's V pieces are the A operands of the identity product,
  // row 16 mt + l16 of the tile at columns 4 g4 .. + 3 of the wave's 16 (one
  // 8-byte load per row tile; rows past the tree and pieces past d_v read row
  // T-1 / column 0 and are zeroed).
  using VC = VTileCfg<DT>;
  using VElem = std::conditional_t<DT == BOLE_BF16, uint16_t, uint32_t>;
  const bool vvec = vecf & kVecV;
  u16x8 vpc[VC::PER];
  bf16x4 va[4];
  if (EARLY) {
    const int c4 = kBV * r + 16 * w + 4 * g4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 16 * mt + l16;
      const bool in = row < T && c4 < d_v;
      const int64_t e =
          ((int64_t)(off + rowNode[min(row, T - 1)]) * H + h) * d_v + (c4 < d_v ? c4 : 0);
      const u16x4 raw = *reinterpret_cast<const u16x4*>(reinterpret_cast<const uint16_t*>(v) + e);
      va[mt] = __builtin_bit_cast(bf16x4, in ? raw : u16x4{0, 0, 0, 0});
    }
  } else {
    const u16x8* vsafe = reinterpret_cast<const u16x8*>(reinterpret_cast<uintptr_t>(v) & ~uintptr_t(15));
#pragma unroll
    for (int it = 0; it < VC::PER; ++it) {
      const int id = threadIdx.x + kThreads * it;
      const int row = id / VC::PPR, col = kBV * r + VC::EPP * (id % VC::PPR);
      const bool in = row < T && col < d_v;
      const int64_t e =
          ((int64_t)(off + rowNode[min(row, T - 1)]) * H + h) * d_v + (col < d_v ? col : 0);
      const u16x8* src = vvec ? reinterpret_cast<const u16x8*>(reinterpret_cast<const VElem*>(v) + e)
                              : vsafe;
      const u16x8 val = *src;
      vpc[it] = in ? val : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  f32x4 qs[4], ks[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    qs[mt] = zero_f32x4();
    ks[mt] = zero_f32x4();
  }
  constexpr bool kOne = FUSED || ONE;
  for (int kc0 = 0; kc0 < (kOne ? 1 : d_k); kc0 += SC::KC) {
    if (!kOne && kc0 > 0) {
      __syncthreads();  // every wave is done with the previous chunk
      load_s(kc0, 0, kSChunks);
      qk_issue<DT>(qkbuf, q, k, rowNode, T, off, H, h, d_k, kc0);
      qk_commit<DT>(stage, qkbuf);
      __syncthreads();
    }
#pragma unroll
    for (int kk = 0; kk < SC::KC / 32; ++kk) {
      if (COMMIT && pend && kk == 0) {  // uniform
        // the committed state replaces S_pre in the lane's registers and goes
        // back into the slot: the first half of the row chunks now, the second
        // when phase A reaches it (so phase A on the first half overlaps the
        // second half's arrival).  A path longer than 16 nodes takes every
        // step on all chunks here.
        pc.apply(sx, 0, kSHalf, true, cbh, cbl, l16, g4, d_k, ktile);
        if (pc.La > 16) {
          pc.apply(sx, kSHalf, kSChunks, true, cbh, cbl, l16, g4, d_k, ktile);
          // the gate sums again (not held through the main path)
          pc.lp = cm.logP[(int64_t)(po + min(lane, pT - 1)) * H + h];
          pc.lpa = __shfl(pc.lp, pa);
          pc.steps(sx, ktile, 16, vin, g4, l16, d_k);
          pc.store(cbase, sx, 0, kSChunks, cvl, l16, g4, d_k);
        } else {
          pc.store(cbase, sx, 0, kSHalf, cvl, l16, g4, d_k);
        }
      }
      if (COMMIT && pend && kk == kSHalf && pc.La <= 16) {  // uniform
        pc.apply(sx, kSHalf, kSChunks, true, cbh, cbl, l16, g4, d_k, ktile);
        pc.store(cbase, sx, kSHalf, kSChunks, cvl, l16, g4, d_k);
      }
      if (kc0 + 32 * kk < d_k) {
        bf16x8 b_hi, b_lo;
        split_bf16x8(sx[kk], b_hi, b_lo);
        // every row tile runs: staged rows past the tree are zero, and a
        // per-tile branch would cost a copy of every accumulator at its join
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = 16 * mt + l16;
          const int ro = row * SC::LROW + 8 * swz<DT>(row, 4 * kk + g4);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(stage + ro);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(stage + kMaxTree * SC::LROW + ro);
          // B0 = D_P Q S feeds only O, and keeps S's low half all the same:
          // taken on the hi parts only, O's own products lose about 2^-9 of
          // each term, and where B0 and C U nearly cancel (beta near 1, q
          // close to k, a state large against v) that is no longer small
          // against O (the 2e-2 bar was missed with states 100x the spread
          // of prefix-built ones)
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
  if (!EARLY) __syncthreads();  // diagonal inverses visible; staged Q/K rows no longer read
  // Past this point the wave holds all its inputs and only its tail is left:
  // it takes issue priority over waves still in their load phases (the two
  // workgroups of a CU otherwise finish about 3 us apart at the target shape;
  // measured 0.6 us faster).  Wave priority only orders issue among resident
  // waves.
  __builtin_amdgcn_s_setprio(2);

  // V tile into LDS (over the staged rows); EARLY: V in the accumulator layout
  // by D = V_tile x I on v_mfma_f32_16x16x16_bf16 (exact: one bf16 product
  // with 1.0 per entry), the lane's rows 16 mt + 4 g4 + e of column vloc
  VElem* vt = reinterpret_cast<VElem*>(stage);
  f32x4 vacc[4];
  if (EARLY) {
    bf16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (__bf16)(4 * g4 + e == l16 ? 1.0f : 0.0f);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vacc[mt] = mfma16_bf16(va[mt], ident, zero_f32x4());
  } else if (vvec) {
#pragma unroll
    for (int it = 0; it < VC::PER; ++it) {
      const int id = threadIdx.x + kThreads * it;
      const int row = id / VC::PPR, c = VC::EPP * (id % VC::PPR);
      *reinterpret_cast<u16x8*>(vt + vtile_idx(row, c)) = vpc[it];
    }
  } else {
    for (int it = 0; it < kMaxTree * kBV / kThreads; ++it) {
      const int id = threadIdx.x + kThreads * it;
      const int row = id / kBV, c = id % kBV, col = kBV * r + c;
      VElem x = 0;
      if (row < T && col < d_v)
        x = reinterpret_cast<const VElem*>(v)[((int64_t)(off + rowNode[row]) * H + h) * d_v + col];
      vt[vtile_idx(row, c)] = x;
    }
  }
  if (!EARLY) __syncthreads();  // V tile visible

  // B0 = D_P QS, R = D_beta (V - D_P KS); rows beyond the tree are exact zeros.
  f32x4 ru[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 16 * mt + 4 * g4 + e;
      const float P = rowP[p], bt = rowBeta[p];
      float vx;
      if (EARLY) {
        vx = vacc[mt][e];
      } else {
        const VElem raw = vt[vtile_idx(p, vloc)];
        vx = __builtin_bit_cast(float, DT == BOLE_BF16 ? (uint32_t)raw << 16 : (uint32_t)raw);
      }
      qs[mt][e] = P * qs[mt][e];
      ru[mt][e] = bt * (vx - P * ks[mt][e]);
    }
  }

  f32x4 u[4];
  if (SOLVE == kSolveBlocked) {
    // ---------------- Solve (I + G) U = R by 16-row tiles --------------------
    // U_t = (I + G_tt)^-1 (R_t - sum_{s<t} G_ts U_s).  The sum uses the 32-wide
    // permuted blocks of -G with the tiles not yet solved entered as zeros; the
    // lane's own U tiles are the B operand.  Tiles past the tree stay zero.
#pragma unroll
    for (int t = 0; t < 4; ++t) u[t] = zero_f32x4();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nmt) {
        f32x4 y = ru[t];
#pragma unroll
        for (int J = 0; J <= t / 2; ++J) {
          if (2 * J < t) {  // block J holds a solved tile
            bf16x8 zh, zl;
            split_pair(u[2 * J], 2 * J + 1 < t ? u[2 * J + 1] : zero_f32x4(), zh, zl);
            const int o = gc_frag(16 * t + l16, J, g4);
            const bf16x8 gh = *reinterpret_cast<const bf16x8*>(gcs + o);
            const bf16x8 gl = *reinterpret_cast<const bf16x8*>(gcs + kGcPlane + o);
            y = mfma_bf16(gh, zh, y);
            y = mfma_bf16(gl, zh, y);
            y = mfma_bf16(gh, zl, y);
          }
        }
        bf16x4 yh, yl;
        split_bf16x4(y, yh, yl);
        const bf16x4 ih = invs[t][0][lane], il = invs[t][1][lane];
        f32x4 acc = mfma16_bf16(ih, yh, zero_f32x4());
        acc = mfma16_bf16(il, yh, acc);
        u[t] = mfma16_bf16(ih, yl, acc);
      }
    }

  } else if (SOLVE == kSolveNeumann) {
    // ------------- Neumann propagation: Z <- -G Z, U += Z, d_b steps -------------
    // The product uses the same permuted 32-wide blocks of -G as the
    // substitution (entries above the diagonal are zero), with the lane's own Z
    // tiles as the B operand.  Tile depth bounds are uniform across the
    // workgroup: the rows are shared, so no wave diverges.
    int tmax[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) tmax[t] = 16 * t < T ? rowDep[min(16 * t + 15, T - 1)] : -1;
    // level order: the last row is the deepest (at most T - 1 in a valid tree;
    // the bound keeps the loop short whatever the depth input holds)
    const int dmax = min(rowDep[T - 1], T - 1);
    // B0 waits in LDS while the propagation runs, at the lane's own positions
    // of the U tile that is written there later (held in registers across the
    // loop it would spill).  The V tile shares those bytes: every wave must be
    // done reading it first.
    float* park = reinterpret_cast<float*>(stage);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) park[vtile_idx(16 * t + 4 * g4 + e, vloc)] = qs[t][e];
    asm volatile("" ::: "memory");
    f32x4 z[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u[t] = ru[t];
      z[t] = ru[t];
    }
    for (int m = 1; m <= dmax; ++m) {
      bf16x8 zh[2], zl[2];
#pragma unroll
      for (int J = 0; J < 2; ++J) split_pair(z[2 * J], z[2 * J + 1], zh[J], zl[J]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 y = zero_f32x4();
        if (tmax[I] >= m) {
#pragma unroll
          for (int J = 0; J <= I / 2; ++J) {
            if (max(tmax[2 * J], tmax[2 * J + 1]) >= m - 1) {
              // re-read every step: held across the loop, the six blocks of
              // -G would take 48 registers and spill
              int o = gc_frag(16 * I + l16, J, g4);
              asm volatile("" : "+v"(o));
              const bf16x8 gh = *reinterpret_cast<const bf16x8*>(gcs + o);
              const bf16x8 gl = *reinterpret_cast<const bf16x8*>(gcs + kGcPlane + o);
              y = mfma_bf16(gh, zh[J], y);
              y = mfma_bf16(gl, zh[J], y);
              y = mfma_bf16(gh, zl[J], y);
            }
          }
        }
        z[I] = y;
        u[I] += y;
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) qs[t][e] = park[vtile_idx(16 * t + 4 * g4 + e, vloc)];
  } else {
    // ------------- Inverse: U = W R, O = B0 + M R -------------
    bf16x8 rh[2], rl[2];
#pragma unroll
    for (int J = 0; J < 2; ++J) split_pair(ru[2 * J], ru[2 * J + 1], rh[J], rl[J]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 y = zero_f32x4(), acc = qs[I];
      if (I < nmt) {
#pragma unroll
        for (int J = 0; J <= I / 2; ++J) {
          const int o = gc_frag(16 * I + l16, J, g4);
          const bf16x8 wh = *reinterpret_cast<const bf16x8*>(gcs + o);
          const bf16x8 wl = *reinterpret_cast<const bf16x8*>(gcs + kGcPlane + o);
          const bf16x8 mh = *reinterpret_cast<const bf16x8*>(gcs + 2 * kGcPlane + o);
          y = mfma_bf16(wh, rh[J], y);
          y = mfma_bf16(wl, rh[J], y);
          y = mfma_bf16(wh, rl[J], y);
          acc = mfma_bf16(mh, rh[J], acc);
          const bf16x8 ml = *reinterpret_cast<const bf16x8*>(gcs + 3 * kGcPlane + o);
          acc = mfma_bf16(ml, rh[J], acc);
          acc = mfma_bf16(mh, rl[J], acc);
        }
      }
      u[I] = y;
      qs[I] = acc;
    }
  }
  if (SOLVE != kSolveInverse) {
    // ---------------- Readout: O = B0 + C U ----------------
    bf16x8 uh[2], ul[2];
#pragma unroll
    for (int J = 0; J < 2; ++J) split_pair(u[2 * J], u[2 * J + 1], uh[J], ul[J]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc = qs[I];  // plane rows past tile nmt are zero
#pragma unroll
      for (int J = 0; J <= I / 2; ++J) {
        const int o = gc_frag(16 * I + l16, J, g4);
        const bf16x8 ch = *reinterpret_cast<const bf16x8*>(gcs + 2 * kGcPlane + o);
        const bf16x8 cl = *reinterpret_cast<const bf16x8*>(gcs + 3 * kGcPlane + o);
        acc = mfma_bf16(ch, uh[J], acc);
        acc = mfma_bf16(cl, uh[J], acc);
        acc = mfma_bf16(ch, ul[J], acc);
      }
      qs[I] = acc;
    }
  }

  // ---------------- Store U and O through LDS ----------------
  // The tiles are written to LDS in the accumulator layout and leave as 4-element
  // pieces of the nodes' rows (16 bytes of U, 8 or 16 of O per lane).
  using OElem = std::conditional_t<DT == BOLE_BF16, uint16_t, float>;
  __syncthreads();  // every wave is done with the staged rows, the V tile and the C planes
  float* ut = reinterpret_cast<float*>(stage);
  OElem* ot = reinterpret_cast<OElem*>(gcs);
#pragma unroll
  for (int I = 0; I < 4; ++I) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = vtile_idx(16 * I + 4 * g4 + e, vloc);
      ut[idx] = u[I][e];
      if (DT == BOLE_BF16)
        ot[idx] = float_to_bf16_bits(qs[I][e]);
      else
        ot[idx] = qs[I][e];
    }
  }
  __syncthreads();  // output tiles visible
  if (vecf & kVecOut) {
#pragma unroll
    for (int it = 0; it < kMaxTree * kBV / 4 / kThreads; ++it) {
      const int id = threadIdx.x + kThreads * it;
      const int row = id / (kBV / 4), c = 4 * (id % (kBV / 4)), col = kBV * r + c;
      if (row < T && col < d_v) {
        const int64_t at = ((int64_t)(off + rowNode[row]) * H + h) * d_v + col;
        const int idx = vtile_idx(row, c);
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(ut + idx),
                                    reinterpret_cast<f32x4*>(U + at));
        if (DT == BOLE_BF16)
          __builtin_nontemporal_store(*reinterpret_cast<const u16x4*>(ot + idx),
                                      reinterpret_cast<u16x4*>(reinterpret_cast<uint16_t*>(O) + at));
        else
          __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(ot + idx),
                                      reinterpret_cast<f32x4*>(reinterpret_cast<float*>(O) + at));
      }
    }
  } else {
    for (int it = 0; it < kMaxTree * kBV / kThreads; ++it) {
      const int id = threadIdx.x + kThreads * it;
      const int row = id / kBV, c = id % kBV, col = kBV * r + c;
      if (row < T && col < d_v) {
        const int64_t at = ((int64_t)(off + rowNode[row]) * H + h) * d_v + col;
        const int idx = vtile_idx(row, c);
        U[at] = ut[idx];
        reinterpret_cast<OElem*>(O)[at] = ot[idx];
      }
    }
  }
}

}  // namespace bole

namespace {
template <int DT, bool FUSED, bool ONE, bool PREP = false, int SOLVE = bole::kSolveBlocked,
          bool COMMIT = false>
int launch_verify_t(const void* q, const void* k, const void* v, const float* logP,
                    const float* beta, const float* state_pool, int32_t n_slots,
                    const int32_t* slot, const float* G, const float* C, const uint64_t* anc,
                    const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                    const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                    int32_t d_v, void* O, float* U, uint32_t* err, hipStream_t s,
                    bole::PrepIO prep = bole::PrepIO{}, bole::CommitIO cm = bole::CommitIO{}) {
  const int NV = (d_v + bole::kBV - 1) / bole::kBV;
  const dim3 block(bole::kThreads);
  const int esize = DT == BOLE_BF16 ? 2 : 4;
  const bool v_ok = d_v % (16 / esize) == 0 && (uintptr_t)v % 16 == 0;
  const bool out_ok = d_v % 4 == 0 && (uintptr_t)U % 16 == 0 && (uintptr_t)O % (4 * esize) == 0;
  const int vecf = (v_ok ? bole::kVecV : 0) | (out_ok ? bole::kVecOut : 0);
  // the early tail (fused producer only: without Gram work, half the waves
  // would wait at its barrier) reads V as 8-byte pieces of four columns
  constexpr bool kMayEarly = DT == BOLE_BF16 && SOLVE == bole::kSolveBlocked && FUSED;
  const bool early = kMayEarly && d_v % 4 == 0 && (uintptr_t)v % 8 == 0;
  // One launch whatever the grid: a grid beyond one residency round (two
  // workgroups per CU) starts its later workgroups as earlier ones finish, so
  // their loads overlap the earlier ones' tails and stores.  (Split into
  // back-to-back launches of one round each, 32 requests x 32 heads measured
  // about 10% slower.)
  const dim3 grid(B * H * NV);
  if (early) {
    if constexpr (kMayEarly)
      hipLaunchKernelGGL((bole::verify_kernel<DT, FUSED, ONE, PREP, SOLVE, COMMIT, true>), grid,
                         block, 0, s, q, k, v, logP, beta, state_pool, n_slots, slot, G, C, anc,
                         order, depth, tree_off, tree_depth, B, N, H, d_k, d_v, O, U, vecf, prep,
                         err, cm);
  } else {
    hipLaunchKernelGGL((bole::verify_kernel<DT, FUSED, ONE, PREP, SOLVE, COMMIT>), grid, block, 0,
                       s, q, k, v, logP, beta, state_pool, n_slots, slot, G, C, anc, order, depth,
                       tree_off, tree_depth, B, N, H, d_k, d_v, O, U, vecf, prep, err, cm);
  }
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}

template <bool FUSED, int SOLVE = bole::kSolveBlocked>
int launch_verify(int32_t dtype, const void* q, const void* k, const void* v, const float* logP,
                  const float* beta, const float* state_pool, int32_t n_slots,
                  const int32_t* slot, const float* G, const float* C, const uint64_t* anc,
                  const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                  const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                  int32_t d_v, void* O, float* U, uint32_t* err, hipStream_t s) {
#define BOLE_VERIFY_ARGS                                                                     \
  q, k, v, logP, beta, state_pool, n_slots, slot, G, C, anc, order, depth, tree_off, tree_depth, \
      B, N, H, d_k, d_v, O, U, err, s
  if (dtype == BOLE_BF16) {
    if (FUSED || d_k <= bole::StageCfg<BOLE_BF16>::KC)
      return launch_verify_t<BOLE_BF16, FUSED, true, false, SOLVE>(BOLE_VERIFY_ARGS);
    return launch_verify_t<BOLE_BF16, false, false, false, SOLVE>(BOLE_VERIFY_ARGS);
  }
  if (FUSED || d_k <= bole::StageCfg<BOLE_F32>::KC)
    return launch_verify_t<BOLE_F32, FUSED, true, false, SOLVE>(BOLE_VERIFY_ARGS);
  return launch_verify_t<BOLE_F32, false, false, false, SOLVE>(BOLE_VERIFY_ARGS);
#undef BOLE_VERIFY_ARGS
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

extern "C" int bole_verify_neumann_launch(int32_t dtype, const void* q, const void* k,
                                          const void* v, const float* logP, const float* beta,
                                          const float* state_pool, int32_t n_slots,
                                          const int32_t* slot, const float* G, const float* C,
                                          const int32_t* order, const int32_t* depth,
                                          const int32_t* tree_off, const int32_t* tree_depth,
                                          int32_t B, int32_t N, int32_t H, int32_t d_k,
                                          int32_t d_v, void* O, float* U, uint32_t* err,
                                          hipStream_t s) {
  return launch_verify<false, bole::kSolveNeumann>(dtype, q, k, v, logP, beta, state_pool,
                                                   n_slots, slot, G, C, nullptr, order, depth,
                                                   tree_off, tree_depth, B, N, H, d_k, d_v, O, U,
                                                   err, s);
}

extern "C" int bole_verify_inverse_launch(int32_t dtype, const void* q, const void* k,
                                          const void* v, const float* logP, const float* beta,
                                          const float* state_pool, int32_t n_slots,
                                          const int32_t* slot, const float* W, const float* M,
                                          const int32_t* order, const int32_t* depth,
                                          const int32_t* tree_off, const int32_t* tree_depth,
                                          int32_t B, int32_t N, int32_t H, int32_t d_k,
                                          int32_t d_v, void* O, float* U, uint32_t* err,
                                          hipStream_t s) {
  return launch_verify<false, bole::kSolveInverse>(dtype, q, k, v, logP, beta, state_pool,
                                                   n_slots, slot, W, M, nullptr, order, depth,
                                                   tree_off, tree_depth, B, N, H, d_k, d_v, O, U,
                                                   err, s);
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

extern "C" int bole_tree_verify_launch(int32_t dtype, const void* q, const void* k, const void* v,
                                       const int32_t* parent, const float* log_gamma,
                                       const float* beta, const float* state_pool,
                                       int32_t n_slots, const int32_t* slot,
                                       const int32_t* tree_off, int32_t B, int32_t N, int32_t H,
                                       int32_t d_k, int32_t d_v, void* O, float* U,
                                       int32_t* depth, uint64_t* anc, int32_t* order,
                                       int32_t* tree_depth, float* logP, uint32_t* err,
                                       hipStream_t s) {
  const bole::PrepIO prep{parent, log_gamma, depth, anc, order, tree_depth, logP};
  if (dtype == BOLE_BF16)
    return launch_verify_t<BOLE_BF16, true, true, true>(
        q, k, v, nullptr, beta, state_pool, n_slots, slot, nullptr, nullptr, nullptr, nullptr,
        nullptr, tree_off, nullptr, B, N, H, d_k, d_v, O, U, err, s, prep);
  return launch_verify_t<BOLE_F32, true, true, true>(
      q, k, v, nullptr, beta, state_pool, n_slots, slot, nullptr, nullptr, nullptr, nullptr,
      nullptr, tree_off, nullptr, B, N, H, d_k, d_v, O, U, err, s, prep);
}

extern "C" int bole_commit_tree_verify_launch(
    int32_t dtype, const void* q, const void* k, const void* v, const int32_t* parent,
    const float* log_gamma, const float* beta, float* state_pool, int32_t n_slots,
    const int32_t* slot, const int32_t* tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
    int32_t d_v, void* O, float* U, int32_t* depth, uint64_t* anc, int32_t* order,
    int32_t* tree_depth, float* logP, const void* prev_k, const float* prev_U,
    const float* prev_logP, const uint64_t* prev_anc, const int32_t* prev_tree_off,
    const int32_t* prev_accept, int32_t prev_N, uint32_t* err, hipStream_t s) {
  const bole::PrepIO prep{parent, log_gamma, depth, anc, order, tree_depth, logP};
  const bole::CommitIO cm{state_pool, prev_k,        prev_U,      prev_logP,
                          prev_anc,   prev_tree_off, prev_accept, prev_N};
  if (dtype == BOLE_BF16)
    return launch_verify_t<BOLE_BF16, true, true, true, bole::kSolveBlocked, true>(
        q, k, v, nullptr, beta, state_pool, n_slots, slot, nullptr, nullptr, nullptr, nullptr,
        nullptr, tree_off, nullptr, B, N, H, d_k, d_v, O, U, err, s, prep, cm);
  return launch_verify_t<BOLE_F32, true, true, true, bole::kSolveBlocked, true>(
      q, k, v, nullptr, beta, state_pool, n_slots, slot, nullptr, nullptr, nullptr, nullptr,
      nullptr, tree_off, nullptr, B, N, H, d_k, d_v, O, U, err, s, prep, cm);
}
