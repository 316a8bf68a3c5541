/*
 * bole.h - C ABI of libbole.so: closed-form tree verification for Gated DeltaNet
 * (GDN) layers on AMD MI355X (gfx950).
 *
 * The method is Bole (arXiv 2608.01651, "Bole: Efficient Tree Speculation for
 * Hybrid-Attention Language Models").  For every node of a speculative proposal
 * tree it computes, from one immutable pre-tree state S_pre (Theorem 1, Eq. 2):
 *
 *     O = D_P Q S_pre + C (I + G)^{-1} D_beta (V - D_P K S_pre)
 *
 * with P_i the product of decay gates over node i's root-to-node path (i
 * included), G_ij = beta_i (P_i/P_j) k_i.k_j over strict ancestors j (Lemma 2,
 * Eq. 5), C_ij = (P_i/P_j) q_i.k_j over ancestors-or-self (Eq. 4) and
 * (I+G)^{-1} = sum_{m=0..d} (-G)^m, d the tree depth (Lemma 3, Eq. 6).  After
 * acceptance, the accepted path a is committed as S_new = P_a S_pre +
 * (D_a K_a)^T U_a (Eq. 10).  Equations are numbered as in the paper; the
 * LaTeX of Eqs. 1-12 survives in the xllm-io paper review of the same work.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains them after returning.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously.  Buffers must stay alive until it completes.
 *  - Host-detectable argument errors return a bole_status synchronously and
 *    enqueue nothing.  A failed launch returns BOLE_E_HIP.
 *  - Data-dependent problems found on the device OR bits into *err (a device
 *    uint32; may be NULL to ignore them).  Outputs of an affected tree or state
 *    head are then unspecified, but no kernel writes outside that tree's rows,
 *    that head's G/C tile or that request's state slot.
 *  - Trees: a flat ragged forest.  Tree b owns global node rows
 *    [tree_off[b], tree_off[b+1]); tree sizes are 1..64.  parent[] holds the
 *    LOCAL index of each node's parent inside its tree, -1 for a root.  Any
 *    acyclic labelling is accepted (parents need not precede children).
 *  - Token operands are token-major: q, k [N, H, d_k]; v, O, U [N, H, d_v];
 *    per-node gates [N, H].  Committed states use the serving slot layout
 *    [slot, H, d_v, d_k] (arXiv page, state-lifecycle paragraph), float32.
 *  - d_k and d_v are multiples of 16 in [16, 256].
 *  - Stateless and reentrant: no global state (the one exception is the
 *    per-GPU scratch array of bole_forest_build_noalloc); calls on different
 *    streams may overlap as long as they do not write the same buffers.
 */
#ifndef BOLE_H
#define BOLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BOLE_API __attribute__((visibility("default")))

/* element type of q/k/v (and of O); gates, states, G/C and U are float32 */
typedef enum { BOLE_F32 = 0, BOLE_BF16 = 1 } bole_dtype;

typedef enum {
  BOLE_OK = 0,
  BOLE_E_NULL = 1,        /* a required pointer is NULL */
  BOLE_E_SHAPE = 2,       /* a size is out of range */
  BOLE_E_DTYPE = 3,       /* unknown bole_dtype */
  BOLE_E_UNSUPPORTED = 4, /* d_k / d_v not a multiple of 16 in [16, 256] */
  BOLE_E_HIP = 5          /* a HIP launch failed */
} bole_status;

/* device error bits OR-ed into *err */
#define BOLE_ERR_BAD_PARENT 1u /* parent out of [-1, T_b) or a node its own parent */
#define BOLE_ERR_CYCLE 2u      /* parent links contain a cycle */
#define BOLE_ERR_TREE_SIZE 4u  /* tree_off range empty, larger than 64 or outside [0, N) */
#define BOLE_ERR_BAD_ACCEPT 8u /* accepted node outside [-1, T_b) */
#define BOLE_ERR_BAD_SLOT 16u  /* state slot outside [0, n_slots) */
#define BOLE_ERR_BAD_PROB 32u  /* a draft probability outside [0, 1] or NaN */
#define BOLE_ERR_DISCONNECTED 64u /* a packed node's parent is not an earlier node of its tree */

#define BOLE_MAX_TREE 64

/*
 * bole_tree_prep - round-level topology step plus log-space gate products
 * (arXiv page, section IV-C: a topology step once per round precedes the
 * per-layer GPU stages; review section 三, fused pipeline, stage (1) gate
 * preparation).
 *
 *  in   parent[N]           local parent index per node (-1 = root)
 *  in   tree_off[B+1]       tree row ranges
 *  in   log_gamma[L,N,H]    g = log(gamma) per layer/node/head, or NULL
 *  out  depth[N]            edges to the root (root = 0)
 *  out  anc[N]              ancestor-or-self bit set, bit j = local node j
 *  out  order[N]            per tree, local node ids sorted by (depth, id);
 *                           order[tree_off[b] + p] is the p-th node of tree b
 *  out  tree_depth[B]       max depth d_b of tree b (Lemma 3's d); -1 marks a
 *                           tree that failed validation (consumers skip it)
 *  out  logP[L,N,H]         log P_i = sum of g along the root-to-i path, i
 *                           included, summed in float32 root first from +0.0f
 *                           (one rounding per add, no fused ops); NULL iff
 *                           log_gamma is NULL
 *  out  err                 BAD_PARENT, CYCLE, TREE_SIZE
 * Results are bit-exact (integers and the float32 sums alike).
 */
BOLE_API int bole_tree_prep(const int32_t* parent, const int32_t* tree_off, int32_t B, int32_t N,
                   const float* log_gamma, int32_t L, int32_t H, int32_t* depth, uint64_t* anc,
                   int32_t* order, int32_t* tree_depth, float* logP, uint32_t* err,
                   void* stream);

/* Bytes of the G plus C workspace for B trees and H heads: 2*B*H*64*64*4. */
BOLE_API size_t bole_gc_workspace_bytes(int32_t B, int32_t H);

/*
 * bole_factor_gc - the G/C factor producer, one per (tree, head) (review
 * section 三, stage (2); Eq. 4 and Eq. 5 of the paper).
 *
 *  in   q, k [N,H,d_k]      dtype elements
 *  in   logP[N,H], beta[N,H] float32 (this layer)
 *  in   anc[N], order[N], tree_off[B+1] from bole_tree_prep
 *  out  G, C [B,H,64,64]    float32, indexed by LEVEL-ORDER position: with
 *       i = order[tree_off[b] + p] and j = order[tree_off[b] + q],
 *         G[b,h,p,q] = beta_i exp(logP_i - logP_j) k_i.k_j  for j a strict ancestor of i
 *         C[b,h,p,q] = exp(logP_i - logP_j) q_i.k_j         for j an ancestor of i or i
 *       every other entry (including rows/cols >= T_b) is exactly 0.  Level
 *       order puts parents before children, so G is strictly lower triangular
 *       and C lower triangular (the indexing of the paper's Theorem 1).
 *       Dot products run on bf16 MFMA with float32 accumulation (float32
 *       operands are split into bf16 hi+lo parts).
 *  out  err                 TREE_SIZE
 * G and C are per-layer scratch; they can be reused across layers and rounds.
 */
BOLE_API int bole_factor_gc(int32_t dtype, const void* q, const void* k, const float* logP,
                            const float* beta, const uint64_t* anc, const int32_t* order,
                            const int32_t* tree_off, int32_t B, int32_t N, int32_t H,
                            int32_t d_k, float* G, float* C, uint32_t* err, void* stream);

/*
 * bole_verify - value-tiled solve and readout (arXiv page section IV-B; review
 * Eqs. 7 and 8), one layer.
 *
 * For each (tree b, head h, value tile r) it forms
 *     B0 = D_P Q S_pre^(r),  R = D_beta (V^(r) - D_P K S_pre^(r)),
 * U = (I + G)^-1 R (the value of the finite Neumann polynomial
 * sum_{m=0..d_b} (-G)^m R, reached on chip by blocked forward substitution over
 * 16-row tiles, each diagonal block inverted by its own Neumann series), and
 * reads out O^(r) = B0 + C U.
 * All products run on bf16 MFMA with float32 accumulation; float32 operands
 * (states, G, C, U, and float32 q/k) are split into bf16 hi+lo parts.
 *
 *  in   q, k [N,H,d_k], v [N,H,d_v]   dtype
 *  in   logP[N,H], beta[N,H]          float32
 *  in   state_pool[n_slots,H,d_v,d_k] float32, read only (S_pre is immutable)
 *  in   slot[B]                       state slot of each request
 *  in   G, C [B,H,64,64]              from bole_factor_gc (this layer)
 *  in   order[N], depth[N], tree_off[B+1], tree_depth[B] from bole_tree_prep
 *  out  O [N,H,d_v]                   dtype
 *  out  U [N,H,d_v]                   float32, the compact per-node update u_i
 *  out  err                           TREE_SIZE, BAD_SLOT
 * O and U must not alias any input.
 */
BOLE_API int bole_verify(int32_t dtype, const void* q, const void* k, const void* v, const float* logP,
                const float* beta, const float* state_pool, int32_t n_slots, const int32_t* slot,
                const float* G, const float* C, const int32_t* order, const int32_t* depth,
                const int32_t* tree_off, const int32_t* tree_depth, int32_t B, int32_t N,
                int32_t H, int32_t d_k, int32_t d_v, void* O, float* U, uint32_t* err,
                void* stream);

/*
 * bole_verify_neumann - bole_verify with (I + G)^-1 R evaluated as the d-step
 * Neumann propagation the pages run on chip (review Eq. 8 and Lemma 3; arXiv
 * page section IV-B): Z = U = R, then d_b times Z <- -G Z, U += Z, with d_b =
 * the tree's depth (the deepest row of depth[]).  The result equals
 * bole_verify's up to rounding; the two are alternative exact solves of the
 * same structured system.  Row tiles of Z that are structurally zero at a step
 * (all rows shallower than the step) are skipped.
 *
 *  arguments, outputs and errors as bole_verify.
 */
BOLE_API int bole_verify_neumann(int32_t dtype, const void* q, const void* k, const void* v,
                                 const float* logP, const float* beta, const float* state_pool,
                                 int32_t n_slots, const int32_t* slot, const float* G,
                                 const float* C, const int32_t* order, const int32_t* depth,
                                 const int32_t* tree_off, const int32_t* tree_depth, int32_t B,
                                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O, float* U,
                                 uint32_t* err, void* stream);

/*
 * bole_factor_inverse - the factor producer of an explicit-inverse solve (an
 * exact solve the closed form allows; arXiv page, Theorem 1 discussion).  It
 * forms G and C as bole_factor_gc does, then W = (I + G)^-1 by repeated
 * squaring, W = prod_{k : 2^k <= d_b} (I + (-G)^(2^k)) (the finite Neumann
 * polynomial of Lemma 3 in ceil(log2(d_b + 1)) factors), and M = C W, so that a
 * verify needs only U = W R and O = B0 + M R.
 *
 *  arguments as bole_factor_gc, with the outputs
 *  out  W, M [B,H,64,64]  float32, level-order positions as G and C; W and M
 *       are lower triangular, rows and columns >= T_b are exactly 0.  The
 *       squaring and M's product run on bf16 MFMA with every operand split
 *       hi + lo and float32 accumulation.
 *  out  err               TREE_SIZE
 * W and M take the G/C workspace (bole_gc_workspace_bytes).
 */
BOLE_API int bole_factor_inverse(int32_t dtype, const void* q, const void* k, const float* logP,
                                 const float* beta, const uint64_t* anc, const int32_t* order,
                                 const int32_t* tree_off, int32_t B, int32_t N, int32_t H,
                                 int32_t d_k, float* W, float* M, uint32_t* err, void* stream);

/*
 * bole_verify_inverse - bole_verify for the explicit-inverse solve: with W and M
 * from bole_factor_inverse it forms B0 and R as bole_verify does, then
 * U = W R and O = B0 + M R (two independent products, no chain across row
 * tiles).
 *
 *  arguments as bole_verify, with W and M in place of G and C; outputs and
 *  errors as bole_verify.  tree_depth[] is read only to skip rejected trees.
 */
BOLE_API int bole_verify_inverse(int32_t dtype, const void* q, const void* k, const void* v,
                                 const float* logP, const float* beta, const float* state_pool,
                                 int32_t n_slots, const int32_t* slot, const float* W,
                                 const float* M, const int32_t* order, const int32_t* depth,
                                 const int32_t* tree_off, const int32_t* tree_depth, int32_t B,
                                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O, float* U,
                                 uint32_t* err, void* stream);

/*
 * bole_factor_verify - bole_factor_gc and bole_verify in one launch.  With
 * d_v <= 128 a head's value columns form one workgroup, so the factors have a
 * single consumer; here the Gram products and their masked epilogue run inside
 * the verify workgroup from the Q/K rows it stages anyway, and G/C never touch
 * memory.  The arithmetic is the same as the two-call path, so O and U are
 * bit-identical to bole_factor_gc followed by bole_verify.
 *
 *  arguments as bole_verify, with anc[N] (from bole_tree_prep) in place of G, C.
 *  d_k must not exceed 128 for bf16 and 64 for float32 token inputs
 *  (BOLE_E_UNSUPPORTED otherwise; the two-call path has no such limit).
 */
BOLE_API int bole_factor_verify(int32_t dtype, const void* q, const void* k, const void* v,
                                const float* logP, const float* beta, const float* state_pool,
                                int32_t n_slots, const int32_t* slot, const uint64_t* anc,
                                const int32_t* order, const int32_t* depth,
                                const int32_t* tree_off, const int32_t* tree_depth, int32_t B,
                                int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O, float* U,
                                uint32_t* err, void* stream);

/*
 * bole_tree_verify - bole_tree_prep (for one layer) and bole_factor_verify in
 * one launch.  Each (tree, head) workgroup derives its tree's topology and its
 * head's gate sums logP itself, with the arithmetic of bole_tree_prep (so they
 * are bit-identical to it), and publishes them for bole_commit_path: depth,
 * anc, order and tree_depth from head 0, logP from every head.  The
 * per-round topology step and the per-layer gate preparation (arXiv page:
 * the round's stages; review, Eq. 4 paragraph) then cost no launch of their
 * own.
 *
 *  in   q, k, v, beta, state_pool, slot, tree_off, B, N, H, d_k, d_v
 *                                    as bole_factor_verify
 *  in   parent[N]                    local parent of each node, -1 for a root
 *  in   log_gamma[N,H]               float32 log-gates g of this layer
 *  out  O, U                         as bole_factor_verify
 *  out  depth[N], anc[N], order[N], tree_depth[B], logP[N,H]
 *                                    as bole_tree_prep (logP of this layer)
 *  out  err                          BAD_PARENT, CYCLE, TREE_SIZE, BAD_SLOT
 * A rejected tree gets tree_depth -1 and no O or U.  The d_k limit of
 * bole_factor_verify applies.
 */
BOLE_API int bole_tree_verify(int32_t dtype, const void* q, const void* k, const void* v,
                              const int32_t* parent, const float* log_gamma, const float* beta,
                              const float* state_pool, int32_t n_slots, const int32_t* slot,
                              const int32_t* tree_off, int32_t B, int32_t N, int32_t H,
                              int32_t d_k, int32_t d_v, void* O, float* U, int32_t* depth,
                              uint64_t* anc, int32_t* order, int32_t* tree_depth, float* logP,
                              uint32_t* err, void* stream);

/*
 * bole_commit_tree_verify - the previous round's accepted-path commit of this
 * layer (bole_commit_path's update, Eq. 10 of the paper) followed by
 * bole_tree_verify of this round, in one launch.  In a serving loop a layer's
 * commit only has to land before that layer's next verify, so it is deferred
 * to it: each (tree, head) workgroup reads its slot state once, applies the
 * previous round's path update in registers, writes the committed state back
 * and verifies the new tree against it.  The state pool is read and written
 * once per round instead of three times (verify read, commit read and write).
 *
 * Request b of this round is request b of the previous round, in the same
 * slot[b].  The committed state equals bole_commit_path's bit for bit (the
 * same MFMA steps on the same operands), so the outputs equal those of
 * bole_commit_path followed by bole_tree_verify.
 *
 *  in     q, k, v, parent, log_gamma, beta, slot, tree_off, B, N, H, d_k, d_v
 *                                 as bole_tree_verify (this round)
 *  in/out state_pool[n_slots,H,d_v,d_k]  float32, committed in place
 *  out    O, U, depth, anc, order, tree_depth, logP   as bole_tree_verify
 *  in     prev_k[prev_N,H,d_k]    dtype, the previous round's keys of this layer
 *                                 (8-byte aligned)
 *  in     prev_U[prev_N,H,d_v]    float32, the previous round's U of this layer
 *  in     prev_logP[prev_N,H]     float32, its gate sums of this layer
 *  in     prev_anc[prev_N]        the previous forest's ancestor-or-self sets
 *  in     prev_tree_off[B+1]      the previous forest's offsets
 *  in     prev_accept[B]          accepted local node of the previous tree, or
 *                                 -1: nothing to commit for request b
 *  out    err                     as bole_tree_verify, plus TREE_SIZE and
 *                                 BAD_ACCEPT for the previous round's data
 * A rejected new tree still gets its request's commit; a rejected commit
 * (bad previous range or accepted node) leaves the slot unchanged and the
 * verify reads it as it is.  The previous round's buffers must not alias this
 * round's outputs.  The d_k limit of bole_factor_verify applies.
 */
BOLE_API int bole_commit_tree_verify(int32_t dtype, const void* q, const void* k, const void* v,
                                     const int32_t* parent, const float* log_gamma,
                                     const float* beta, float* state_pool, int32_t n_slots,
                                     const int32_t* slot, const int32_t* tree_off, int32_t B,
                                     int32_t N, int32_t H, int32_t d_k, int32_t d_v, void* O,
                                     float* U, int32_t* depth, uint64_t* anc, int32_t* order,
                                     int32_t* tree_depth, float* logP, const void* prev_k,
                                     const float* prev_U, const float* prev_logP,
                                     const uint64_t* prev_anc, const int32_t* prev_tree_off,
                                     const int32_t* prev_accept, int32_t prev_N, uint32_t* err,
                                     void* stream);

/*
 * bole_tree_conv - tree-parallel short causal convolution, the first per-layer
 * stage of the fused tree pipeline, with the bias and SiLU applied in the same
 * pass (arXiv page, sections II-A and IV-C; review page, fused-pipeline
 * paragraph).
 *
 * Node i's window is the last W entries of its request's committed conv state
 * (the W - 1 inputs that preceded the tree, oldest first) followed by the
 * inputs along i's root-to-node path; every root of a tree starts from that
 * state.  Per channel c:
 *     y[i][c] = silu(bias[c] + sum_{j<W} weight[c][j] * window_i[j][c]),
 * tap W-1 multiplying node i's own input.  float32 arithmetic.
 *
 *  in   x[N,C]                         dtype, the node inputs (channels contiguous)
 *  in   weight[C,W], bias[C] or NULL   float32
 *  in   conv_state[n_slots,W-1,C]      dtype, oldest row first (unused when W == 1)
 *  in   slot[B], parent[N], tree_off[B+1]
 *  out  y[N,C]                         dtype; must not alias x
 *  out  err                            BAD_PARENT, CYCLE, TREE_SIZE, BAD_SLOT
 * Requires 1 <= W <= 8, C a multiple of 8 and x, y, conv_state 16-byte aligned
 * (BOLE_E_UNSUPPORTED otherwise).  A rejected tree gets no outputs.
 */
BOLE_API int bole_tree_conv(int32_t dtype, const void* x, const float* weight, const float* bias,
                            const void* conv_state, int32_t n_slots, const int32_t* slot,
                            const int32_t* parent, const int32_t* tree_off, int32_t B, int32_t N,
                            int32_t C, int32_t W, void* y, uint32_t* err, void* stream);

/*
 * bole_conv_commit - the accepted path's conv state, in place: slot[b]'s state
 * becomes the last W - 1 entries of itself followed by the inputs along the
 * path root..accept[b]; accept[b] == -1 leaves it bit-unchanged.  (The
 * counterpart of bole_commit_path for the convolution's short state.)
 *
 *  in/out conv_state[n_slots,W-1,C]  dtype
 *  in     slot[B], x[N,C] (the round's conv inputs), parent[N], tree_off[B+1], accept[B]
 *  out    err                        BAD_PARENT, CYCLE, TREE_SIZE, BAD_ACCEPT, BAD_SLOT
 * With W == 1 there is no state (conv_state may be NULL) and nothing is launched.
 */
BOLE_API int bole_conv_commit(int32_t dtype, void* conv_state, int32_t n_slots,
                              const int32_t* slot, const void* x, const int32_t* parent,
                              const int32_t* tree_off, const int32_t* accept, int32_t B, int32_t N,
                              int32_t C, int32_t W, uint32_t* err, void* stream);

/*
 * bole_commit_path - accepted-path state reconstruction for L layers in one
 * launch, in place (paper Eq. 10; review: unified cross-layer state commit).
 *
 * For each layer l, request b and head h, with a = accept[b] and the path
 * A(a)+{a}:
 *     S[v][c] <- exp(logP_a) S[v][c] + sum_j exp(logP_a - logP_j) U_j[v] k_j[c]
 * The path outer products run on bf16 MFMA with float32 accumulation
 * (float32 operands split into bf16 hi+lo parts).  accept[b] == -1 leaves the
 * slot bit-unchanged.
 *
 *  in/out state_pool + l*state_layer_stride : [n_slots,H,d_v,d_k] float32
 *  in     k + l*k_layer_stride              : [N,H,d_k] dtype
 *  in     U + l*u_layer_stride              : [N,H,d_v] float32
 *  in     logP + l*logp_layer_stride        : [N,H] float32
 *  in     slot[B], anc[N], tree_off[B+1], accept[B] (local node or -1)
 *  out    err                               TREE_SIZE, BAD_ACCEPT, BAD_SLOT
 * Strides are in elements.  Must not run concurrently with a verify that reads
 * the same slots (order them on one stream).  Two requests must not share a
 * slot.
 */
BOLE_API int bole_commit_path(int32_t L, float* state_pool, int64_t state_layer_stride, int32_t n_slots,
                     const int32_t* slot, int32_t dtype, const void* k, int64_t k_layer_stride,
                     const float* U, int64_t u_layer_stride, const float* logP,
                     int64_t logp_layer_stride, const uint64_t* anc, const int32_t* tree_off,
                     const int32_t* accept, int32_t B, int32_t N, int32_t H, int32_t d_k,
                     int32_t d_v, uint32_t* err, void* stream);

/*
 * bole_forest_build - budget selection and the packed-forest builder (review
 * page, section 三: the hardware-aware verification budget and the SGLang
 * integration paragraphs).  Each drafted candidate v is scored with its path's
 * cumulative draft probability rho(v) = prod over the root-to-v path of
 * p_draft(u | parent(u)), taken as a float32 running product root first
 * (rho(root) = p_draft(root)).  Candidates are ranked by rho descending, then
 * depth, request and candidate index ascending, and taken in that order while
 * the forest holds fewer than `capacity` nodes and the request fewer than
 * `max_tree`.  With 0 <= p <= 1 a child never outranks its parent, so every
 * request's selection is prefix-connected (checked: DISCONNECTED).  A request's
 * selected nodes are numbered in rank order (root 0, parents first) and the
 * requests packed in order: the result is the parent / tree_off input of
 * bole_tree_prep and the verify calls.
 *
 *  in   cand_parent[M_total]  local parent of each candidate within its
 *                             request's candidate tree, -1 for the root
 *  in   p_draft[M_total]      float32 conditional draft probability (root: the
 *                             token the request already holds, normally 1)
 *  in   cand_off[B+1]         request b owns candidates [cand_off[b],
 *                             cand_off[b+1]), at most 1024 of them
 *  in   capacity, max_tree    forest capacity (>= 1) and per-request limit
 *                             (1..64)
 *  out  rho[M_total]          float32 score of every candidate (0 for a
 *                             rejected request)
 *  out  parent[capacity]      local parent of each packed node, -1 for roots
 *                             and for slots past the last node
 *  out  cand_of[capacity]     global candidate index of each packed node, -1
 *                             past the last node
 *  out  tree_off[B+1]         packed forest offsets (a request with no node
 *                             gets an empty range)
 *  in   workspace             bole_forest_workspace_bytes(B, max_tree) bytes
 *                             of device scratch, 8-byte aligned
 *  out  err                   BAD_PARENT, CYCLE, BAD_PROB, TREE_SIZE (more
 *                             than 1024 candidates or offsets out of range):
 *                             that request contributes no node; DISCONNECTED
 * Limits: 1 <= B <= 4095, B * max_tree <= 16384 (BOLE_E_SHAPE otherwise).
 * Two launches (per-request scoring and ranking, then one workgroup for the
 * global cut and the packing).
 */
BOLE_API size_t bole_forest_workspace_bytes(int32_t B, int32_t max_tree);
BOLE_API int bole_forest_build(const int32_t* cand_parent, const float* p_draft,
                               const int32_t* cand_off, int32_t B, int32_t M_total,
                               int32_t capacity, int32_t max_tree, float* rho, int32_t* parent,
                               int32_t* cand_of, int32_t* tree_off, void* workspace,
                               uint32_t* err, void* stream);

/*
 * bole_forest_build_noalloc - bole_forest_build for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same selection, packing, outputs and
 * error bits, bit for bit, from the same kernels; the workspace is a fixed
 * device array inside the library (192 KiB per GPU, held until the process
 * ends) instead of an argument.  Nothing is allocated or freed: the array's
 * device address is looked up once per GPU, on the first call made with that
 * GPU current.
 *
 *  arguments, outputs and errors as bole_forest_build, without `workspace`.
 *  Limits as bole_forest_build (B * max_tree <= 16384 is exactly the array's
 *  capacity); BOLE_E_SHAPE beyond them, BOLE_E_HIP if the runtime cannot
 *  name the current device or the array's address.
 * Every call on one GPU uses that GPU's single array: calls that overlap on
 * one GPU (concurrent streams, or host threads) race and must be serialised
 * by the caller.  `stream` must belong to the current device.
 */
BOLE_API int bole_forest_build_noalloc(const int32_t* cand_parent, const float* p_draft,
                                       const int32_t* cand_off, int32_t B, int32_t M_total,
                                       int32_t capacity, int32_t max_tree, float* rho,
                                       int32_t* parent, int32_t* cand_of, int32_t* tree_off,
                                       uint32_t* err, void* stream);

/* Static description of a bole_status code. */
BOLE_API const char* bole_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* BOLE_H */
