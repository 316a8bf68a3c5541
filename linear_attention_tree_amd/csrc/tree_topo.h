// Round-level topology of one proposal tree, derived by a single wave64 (one
// lane per node).  Shared by tree preparation and the verify kernel that does
// its own preparation, so both produce the same depth, ancestor mask and level
// order.
//
// (arXiv page of Bole: ancestor mask; review, Lemma 3's depth d.)  The
// ancestor-or-self set is built by pointer jumping: after round s every lane
// knows the first 2^s nodes of its upward path and the node 2^s steps up; six
// rounds cover any path of a tree with at most 64 nodes, so a lane that still
// has a jump target after six rounds lies on or leads into a cycle.  The level
// order sorts nodes by (depth, local id).
#pragma once

#include "common.h"

namespace bole {

struct TreeTopo {
  int dep;        // depth of node `lane` (-1 past the tree)
  uint64_t anc;   // ancestor-or-self set of node `lane` (local ids)
  int pos;        // level-order position of node `lane`
  int dmax;       // deepest level of the tree
  uint32_t fail;  // BOLE_ERR_BAD_PARENT or BOLE_ERR_CYCLE, uniform over the wave
};

// Called by every lane of one wave; lane < T holds node `lane` with local
// parent p (-1 for a root).
__device__ __forceinline__ TreeTopo tree_topology(int lane, int T, int p) {
  TreeTopo r{-1, 0ull, 0, 0, 0u};
  const bool live = lane < T;
  p = live ? p : -1;
  const bool bad = live && p != -1 && (p < 0 || p >= T || p == lane);
  if (ballot64(bad)) {
    r.fail = BOLE_ERR_BAD_PARENT;
    return r;
  }
  uint64_t anc = live ? (1ull << lane) : 0ull;
  int jmp = live ? p : -1;
  for (int round = 0; round < 6 && ballot64(jmp >= 0); ++round) {
    const int src = jmp >= 0 ? jmp : lane;
    const uint64_t a2 = __shfl(anc, src);
    const int j2 = __shfl(jmp, src);
    if (jmp >= 0) {
      anc |= a2;
      jmp = j2;
    }
  }
  if (ballot64(live && jmp >= 0)) {
    r.fail = BOLE_ERR_CYCLE;
    return r;
  }
  const int dep = live ? __popcll(anc) - 1 : -1;
  // stable sort by (depth, local id): rank = nodes on shallower levels plus
  // lower ids on the same level.  Every level up to the deepest holds a node
  // (a node's parent is one level up), so the scan ends at T.
  int acc = 0, pos = 0, lev = 0;
  for (; acc < T && lev < kMaxTree; ++lev) {
    const uint64_t m = ballot64(dep == lev);
    if (dep == lev) pos = acc + __popcll(m & ((1ull << lane) - 1ull));
    acc += __popcll(m);
  }
  r.dep = dep;
  r.anc = anc;
  r.pos = live ? pos : lane;
  r.dmax = lev - 1;
  return r;
}

}  // namespace bole
