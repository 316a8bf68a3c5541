// Budget selection and the packed-forest builder (review page, section 三: the
// hardware-aware verification budget and the SGLang integration paragraphs).
// Every drafted candidate v is scored with its path's cumulative draft
// probability rho(v), the product of p_draft(u | parent(u)) over v's
// root-to-node path; the best-scoring candidates across all requests fill the
// capacity, at most max_tree per request; a child never outscores its parent,
// so each request's selection is prefix-connected, and it is packed into one
// flat ragged forest that the verify calls take as is.
//
// rho is a float32 running product taken root first (one rounding per factor).
// Candidates are ordered by the 64-bit key
//     rho bits (63..32) | 1023 - depth (31..22) | 4095 - request (21..10)
//       | 1023 - candidate (9..0),
// larger first: rho descending, then depth, request and candidate ascending.
// For rho >= 0 the float's bits order like its value (a -0.0 score enters the
// key as +0.0), and the key is unique.
//
// Two launches.  forest_score_kernel, one workgroup per request: validation,
// depth and rho level by level, the key, and each candidate's rank within its
// request by counting; the first max_tree keys of the request go to a sorted
// list, each with its parent's position in that list.  forest_pack_kernel, one
// workgroup with every listed key in registers: the capacity-th largest by an
// MSB-first radix select, the per-request counts and their scan, and the
// packed parent / candidate arrays.  A request's nodes are its
// selected candidates in key order, so the root is node 0 and parents come
// first.
#include <mutex>

#include "common.h"

namespace bole {

constexpr int kMaxCand = 1024;  // candidates per request
constexpr int kScoreThreads = 256;
constexpr int kCandPer = kMaxCand / kScoreThreads;
constexpr int kPackThreads = 1024;
constexpr int kMaxRequests = 4095;                  // the key's request field
constexpr int kMaxListed = 16384;                   // B * max_tree
constexpr int kListPer = kMaxListed / kPackThreads;  // listed keys per packing thread
constexpr int kWalk = 16;  // path length a node collects in registers

// A probability of -0.0 passes validation (it compares equal to 0) and makes
// rho -0.0, whose sign bit would put its raw bits above every positive score:
// the key takes rho's value, so both zeros rank as +0.0 (then by depth).  The
// rho reported to the caller keeps the product's own bits.
__device__ __forceinline__ uint64_t cand_key(float rho, int depth, int b, int i) {
  const uint32_t score = rho == 0.0f ? 0u : __float_as_uint(rho);
  return ((uint64_t)score << 32) | ((uint64_t)(1023 - depth) << 22) |
         ((uint64_t)(4095 - b) << 10) | (uint64_t)(1023 - i);
}

// list [B, max_tree]: request b's keys in descending order, 0 past its
// eligible candidates; plist [B, max_tree]: the listed candidate's parent's
// position in the same list (-1 for a root).
__global__ __launch_bounds__(kScoreThreads) void forest_score_kernel(
    const int32_t* __restrict__ cand_parent, const float* __restrict__ p_draft,
    const int32_t* __restrict__ cand_off, int32_t M_total, int32_t max_tree,
    float* __restrict__ rho_out, uint64_t* __restrict__ list, int32_t* __restrict__ plist,
    uint32_t* __restrict__ err) {
  __shared__ int par[kMaxCand];
  __shared__ float pl[kMaxCand];
  __shared__ int settled[kMaxCand];  // round (= depth) at which the node's rho was set, or -1
  __shared__ float rh[kMaxCand];
  // 8 spare entries: the rank loop may read up to 7 keys past the last one
  // (unconditionally, the values discarded), which then stay inside the array
  __shared__ uint64_t key[kMaxCand + 8];
  __shared__ int rkl[kMaxCand];
  __shared__ uint32_t flags;
  __shared__ int progress[3];  // nodes settled per round, rotating

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int o = cand_off[b], e = cand_off[b + 1];
  const int M = e - o;
  uint64_t* lst = list + (int64_t)b * max_tree;
  int32_t* plst = plist + (int64_t)b * max_tree;
  if (o < 0 || e > M_total || M < 0 || M > kMaxCand) {
    for (int r = tid; r < max_tree; r += kScoreThreads) lst[r] = 0ull;
    if (tid == 0) report(err, BOLE_ERR_TREE_SIZE);
    return;  // rho of these candidates is left as it is
  }
  if (tid == 0) {
    flags = 0u;
    progress[0] = progress[1] = progress[2] = 0;
  }
  __syncthreads();

  // load and validate: parents in [-1, M) and not the node itself, p in [0, 1]
  uint32_t my_flags = 0u;
  float pv[kCandPer];
  int pp[kCandPer];
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    const int i = tid + kScoreThreads * k;
    pv[k] = 0.0f;
    pp[k] = -1;
    if (i < M) {
      pp[k] = cand_parent[o + i];
      pv[k] = p_draft[o + i];
      if (pp[k] < -1 || pp[k] >= M || pp[k] == i) my_flags |= 1u;
      if (!(pv[k] >= 0.0f && pv[k] <= 1.0f)) my_flags |= 2u;  // NaN fails both
      par[i] = pp[k];
      pl[i] = pv[k];
      settled[i] = -1;
    }
  }
  if (my_flags) atomicOr(&flags, my_flags);
  __syncthreads();
  const uint32_t f0 = flags;
  uint32_t bits = (f0 & 1u) ? BOLE_ERR_BAD_PARENT : (f0 & 2u) ? BOLE_ERR_BAD_PROB : 0u;

  // depth and rho.  Each node walks up to its root collecting the path's
  // probabilities (at most kWalk steps) and multiplies them root first,
  // rho = fl32(...fl32(p_root * p_1)... * p_i): the same roundings, in the same
  // order, as a parent-then-child recurrence.  A tree with a longer path (or a
  // cycle, whose walk never ends) takes the rounds below instead.
  const int lane = tid & 63, wv = tid >> 6;
  const int kUse = (M + kScoreThreads - 1) / kScoreThreads;  // candidate slots in use
  int dep[kCandPer];
  uint32_t deep = 0u;
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    dep[k] = -1;
    const int i = tid + kScoreThreads * k;
    if (!bits && k < kUse && i < M) {
      float pa[kWalk];
      int j = i, d = -1;
#pragma unroll
      for (int st = 0; st < kWalk; ++st) {
        if (j >= 0) {
          pa[st] = pl[j];
          j = par[j];
          d = st;
        }
      }
      if (j >= 0) {
        deep = 1u;
      } else {
        float x = 0.0f;
#pragma unroll
        for (int st = kWalk - 1; st >= 0; --st) {
          if (st == d) x = pa[st];
          else if (st < d) x = __fmul_rn(x, pa[st]);
        }
        rh[i] = x;
        dep[k] = d;
      }
    }
  }
  if (deep) atomicOr(&flags, 8u);
  __syncthreads();
  if (!bits && (flags & 8u)) {
    // level by level: in round r the nodes whose parent settled in round r - 1
    // settle (the roots in round 0), rho = fl32(rho_parent * p).  A parent
    // settling in the same round reads as -1 or r, never r - 1, so only final
    // values are used.  The rounds stop at the first that settles nothing; a
    // node left unsettled then lies on a cycle.  One barrier per round: the
    // round's counter is read after it, and the counter reset during round r
    // was last read before round r - 1's barrier.
#pragma unroll
    for (int k = 0; k < kCandPer; ++k) dep[k] = -1;
    for (int r = 0; r <= M; ++r) {
      int mine = 0;
#pragma unroll
      for (int k = 0; k < kCandPer; ++k) {
        const int i = tid + kScoreThreads * k;
        if (i < M && dep[k] < 0) {
          const bool go = pp[k] < 0 ? r == 0 : r > 0 && settled[pp[k]] == r - 1;
          if (go) {
            rh[i] = pp[k] < 0 ? pv[k] : __fmul_rn(rh[pp[k]], pv[k]);
            settled[i] = r;
            dep[k] = r;
            ++mine;
          }
        }
      }
      // one counter add per wave
#pragma unroll
      for (int d = 32; d > 0; d >>= 1) mine += __shfl_xor(mine, d);
      if (lane == 0 && mine) atomicAdd(&progress[r % 3], mine);
      if (tid == 0) progress[(r + 1) % 3] = 0;
      __syncthreads();
      if (progress[r % 3] == 0) break;  // uniform: read after the barrier
    }
    uint32_t cyc = 0u;
#pragma unroll
    for (int k = 0; k < kCandPer; ++k) {
      const int i = tid + kScoreThreads * k;
      if (i < M && dep[k] < 0) cyc = 1u;
    }
    if (cyc) atomicOr(&flags, 4u);
    __syncthreads();
    if (flags & 4u) bits = BOLE_ERR_CYCLE;
  }
  if (bits) {
    for (int r = tid; r < max_tree; r += kScoreThreads) lst[r] = 0ull;
    for (int i = tid; i < M; i += kScoreThreads) rho_out[o + i] = 0.0f;
    if (tid == 0) report(err, bits);
    return;
  }

  uint64_t mine[kCandPer];
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    const int i = tid + kScoreThreads * k;
    mine[k] = 0ull;
    if (i < M) {
      mine[k] = cand_key(rh[i], dep[k], b, i);
      key[i] = mine[k];
      rho_out[o + i] = rh[i];
    }
  }
  for (int i = tid; i < M; i += kScoreThreads) rkl[i] = 0;
  __syncthreads();
  // rank within the request: how many of its keys are larger.  Lane l counts
  // for candidates l, l + 64, ... over a quarter of the keys (wave w's), and
  // the four partial counts are added up (broadcast reads, eight at a time).
  {
    constexpr int kSlots = kMaxCand / 64;
    const int nm = (M + 63) / 64;
    const int jq = (M + 3) / 4, j0 = wv * jq, j1 = min(M, j0 + jq);
    uint64_t ck[kSlots];
    int cr[kSlots];
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int c = lane + 64 * m;
      ck[m] = m < nm && c < M ? key[c] : ~0ull;
      cr[m] = 0;
    }
    for (int j = j0; j < j1; j += 8) {
      uint64_t kj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) kj[q] = j + q < j1 ? key[j + q] : 0ull;
#pragma unroll
      for (int m = 0; m < kSlots; ++m)
        if (m < nm)
#pragma unroll
          for (int q = 0; q < 8; ++q) cr[m] += kj[q] > ck[m] ? 1 : 0;
    }
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int c = lane + 64 * m;
      if (m < nm && c < M && cr[m]) atomicAdd(&rkl[c], cr[m]);
    }
  }
  __syncthreads();
  int rk[kCandPer];
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    const int i = tid + kScoreThreads * k;
    rk[k] = i < M ? rkl[i] : 0;
  }
#pragma unroll
  for (int k = 0; k < kCandPer; ++k) {
    const int i = tid + kScoreThreads * k;
    if (i < M && rk[k] < max_tree) {
      // a parent outranks its children, so it is listed too
      lst[rk[k]] = mine[k];
      plst[rk[k]] = pp[k] < 0 ? -1 : rkl[pp[k]];
    }
  }
  for (int r = M + tid; r < max_tree; r += kScoreThreads) lst[r] = 0ull;
}

// One workgroup.  E = B * max_tree listed keys (0 = no candidate), held in
// registers: thread t owns entries t, t + 1024, ...
__global__ __launch_bounds__(kPackThreads) void forest_pack_kernel(
    const int32_t* __restrict__ cand_off, int32_t B, int32_t capacity, int32_t max_tree,
    const uint64_t* __restrict__ list, const int32_t* __restrict__ plist,
    int32_t* __restrict__ parent, int32_t* __restrict__ cand_of, int32_t* __restrict__ tree_off,
    uint32_t* __restrict__ err) {
  __shared__ uint32_t hist[2][256];  // alternate passes: one is cleared while the other fills
  __shared__ uint32_t total, sel_digit, sel_above, sel_count, bad;
  __shared__ unsigned long long kmin;
  __shared__ int wsum[kPackThreads / 64];
  __shared__ int cnt[kMaxRequests + 1];   // selected per request, then tree_off
  __shared__ int coff[kMaxRequests + 1];  // cand_off
  __shared__ uint8_t sel[kMaxListed];     // listed entry selected
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int E = B * max_tree;

  uint64_t kr[kListPer];
  int pr[kListPer];
#pragma unroll
  for (int j = 0; j < kListPer; ++j) {
    const int x = tid + kPackThreads * j;
    kr[j] = x < E ? list[x] : 0ull;
    pr[j] = x < E ? plist[x] : -1;
  }
  for (int b = tid; b <= B; b += kPackThreads) {
    cnt[b] = 0;
    coff[b] = cand_off[b];
  }
  if (tid == 0) {
    total = 0u;
    bad = 0u;
    kmin = ~0ull;
  }
  if (tid < 256) hist[0][tid] = 0u;
  __syncthreads();
  uint32_t c0 = 0u;
#pragma unroll
  for (int j = 0; j < kListPer; ++j) c0 += kr[j] != 0ull ? 1u : 0u;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) c0 += __shfl_xor(c0, d);
  if (lane == 0 && c0) atomicAdd(&total, c0);  // one add per wave
  __syncthreads();

  // the threshold: every listed key >= kstar is selected.  MSB-first radix
  // select of the capacity-th largest listed key (keys are unique), 8 bits a
  // pass; once the chosen digit's keys are exactly the ones still needed, the
  // threshold is the smallest of them and the passes stop.
  uint64_t kstar = 1ull;
  if (total > (uint32_t)capacity) {
    uint64_t prefix = 0ull, mask = 0ull;
    uint32_t need = (uint32_t)capacity;  // still to take among keys matching prefix
    bool settled = false;
    for (int pass = 0; pass < 8 && !settled; ++pass) {
      const int shift = 56 - 8 * pass;
      uint32_t* h = hist[pass & 1];
      // the wave's keys are counted per distinct digit: one add per digit
      // (the high digits are shared by most keys, and same-address adds
      // would serialise)
#pragma unroll
      for (int j = 0; j < kListPer; ++j) {
        const uint64_t k = kr[j];
        bool act = k != 0ull && (k & mask) == prefix;
        const uint32_t dig = (uint32_t)(k >> shift) & 255u;
        uint64_t m = ballot64(act);
        while (m) {
          const int leader = __builtin_ctzll(m);
          const uint32_t dl = (uint32_t)__shfl((int)dig, leader);
          const uint64_t same = ballot64(act && dig == dl);
          if (lane == leader) atomicAdd(&h[dl], (uint32_t)__popcll(same));
          act = act && dig != dl;
          m &= ~same;
        }
      }
      // the other buffer was last read by the previous pass's scan, which
      // ended before that pass's second barrier
      if (tid < 256) hist[(pass & 1) ^ 1][tid] = 0u;
      __syncthreads();
      if (w == 0) {
        // lane l holds digits 255 - 4l .. 252 - 4l; an inclusive scan from the
        // top finds the digit where the count from above reaches need
        uint32_t c[4], sum = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = h[255 - 4 * lane - q];
          sum += c[q];
        }
        uint32_t incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t v = __shfl_up(incl, d);
          if (lane >= d) incl += v;
        }
        uint32_t above = incl - sum;  // keys in higher digits than this lane's
        if (above < need && need <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (above + c[q] >= need) {
              sel_digit = (uint32_t)(255 - 4 * lane - q);
              sel_above = above;
              sel_count = c[q];
              break;
            }
            above += c[q];
          }
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sel_digit << shift;
      mask |= 255ull << shift;
      need -= sel_above;
      settled = sel_count == need;  // uniform
    }
    // every key matching the prefix is selected: the threshold is their minimum
    uint64_t lo = ~0ull;
#pragma unroll
    for (int j = 0; j < kListPer; ++j) {
      const uint64_t k = kr[j];
      if (k != 0ull && (k & mask) == prefix && k < lo) lo = k;
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      const uint64_t v = __shfl_xor(lo, d);
      lo = v < lo ? v : lo;
    }
    if (lane == 0 && lo != ~0ull) atomicMin(&kmin, (unsigned long long)lo);
    __syncthreads();
    kstar = kmin;
  }

  // per-request counts: a request's list is in descending order, so its
  // selected entries are a prefix and the last of them gives the count; then
  // their exclusive scan in place (thread t scans the requests [t * per,
  // t * per + per))
#pragma unroll
  for (int j = 0; j < kListPer; ++j) {
    const int x = tid + kPackThreads * j;
    if (x < E) sel[x] = kr[j] != 0ull && kr[j] >= kstar ? 1 : 0;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kListPer; ++j) {
    const int x = tid + kPackThreads * j;
    if (x < E && sel[x]) {
      const int b = x / max_tree, r = x - (x / max_tree) * max_tree;
      if (r == max_tree - 1 || !sel[x + 1]) cnt[b] = r + 1;
    }
  }
  __syncthreads();
  const int per = (B + kPackThreads - 1) / kPackThreads;
  const int b0 = tid * per, b1 = min(B, b0 + per);
  int my_sum = 0;
  for (int b = b0; b < b1; ++b) my_sum += cnt[b];
  int incl = my_sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = incl - my_sum;
  for (int q = 0; q < w; ++q) base += wsum[q];
  for (int b = b0; b < b1; ++b) {
    const int n = cnt[b];
    cnt[b] = base;  // now tree_off[b]
    tree_off[b] = base;
    base += n;
  }
  __syncthreads();
  if (b0 < B && b1 == B) {  // the owner of the last range closes the offsets
    cnt[B] = base;
    tree_off[B] = base;
  }
  __syncthreads();

  // pack: node r of request b is its r-th listed key
#pragma unroll
  for (int j = 0; j < kListPer; ++j) {
    const int x = tid + kPackThreads * j;
    const uint64_t k = kr[j];
    if (k != 0ull && k >= kstar) {
      const int b = x / max_tree, r = x - (x / max_tree) * max_tree;
      const int pos = cnt[b] + r;
      const int pl = pr[j];
      // prefix connectivity: a non-root's parent is an earlier node of its tree
      const bool root = (k >> 22 & 1023ull) == 1023ull;
      if (root ? pl != -1 : !(pl >= 0 && pl < r)) atomicOr(&bad, 1u);
      if (pos < capacity) {
        cand_of[pos] = coff[b] + (1023 - (int)(k & 1023ull));
        parent[pos] = pl;
      }
    }
  }
  for (int pos = cnt[B] + tid; pos < capacity; pos += kPackThreads) {
    cand_of[pos] = -1;
    parent[pos] = -1;
  }
  if (tid == 0 && bad) report(err, BOLE_ERR_DISCONNECTED);
}

}  // namespace bole

// ---------------------------------------------------------------------------
// Device scratch for bole_forest_build_noalloc: the listed keys and parent
// positions (12 bytes per listed slot) of the largest shape the builder takes,
// B * max_tree = kMaxListed, in a fixed array of 192 KiB that each GPU the
// library runs on holds until the process ends.  Every call on a GPU shares
// that GPU's copy, so calls that overlap on one GPU race; nothing in it has to
// start at zero (the scoring kernel writes every listed slot the packing
// kernel reads).  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
namespace {
constexpr size_t kForestScratchBytes = 12u * (size_t)bole::kMaxListed;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // the array's device address, per device
}  // namespace

static __device__ __align__(256) unsigned char scratch[kForestScratchBytes];

// The device address of the scratch array on the current device (resolved on
// the first call there), for a request of `bytes`.  BOLE_E_SHAPE when it does
// not fit, BOLE_E_HIP when the runtime cannot name the device or the address.
extern "C" int bole_forest_scratch(size_t bytes, void** out) {
  if (bytes > kForestScratchBytes) return BOLE_E_SHAPE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BOLE_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return BOLE_E_HIP;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return BOLE_OK;
}

extern "C" int bole_forest_build_launch(const int32_t* cand_parent, const float* p_draft,
                                        const int32_t* cand_off, int32_t B, int32_t M_total,
                                        int32_t capacity, int32_t max_tree, float* rho,
                                        int32_t* parent, int32_t* cand_of, int32_t* tree_off,
                                        void* workspace, uint32_t* err, hipStream_t s) {
  uint64_t* list = reinterpret_cast<uint64_t*>(workspace);
  int32_t* plist = reinterpret_cast<int32_t*>(list + (int64_t)B * max_tree);
  hipLaunchKernelGGL(bole::forest_score_kernel, dim3(B), dim3(bole::kScoreThreads), 0, s,
                     cand_parent, p_draft, cand_off, M_total, max_tree, rho, list, plist, err);
  if (hipGetLastError() != hipSuccess) return BOLE_E_HIP;
  hipLaunchKernelGGL(bole::forest_pack_kernel, dim3(1), dim3(bole::kPackThreads), 0, s,
                     cand_off, B, capacity, max_tree, list, plist, parent, cand_of, tree_off,
                     err);
  return hipGetLastError() == hipSuccess ? BOLE_OK : BOLE_E_HIP;
}
