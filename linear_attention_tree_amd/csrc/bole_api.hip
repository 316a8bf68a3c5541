// C ABI of libbole: host-side argument validation, then one or two kernel
// launches on the caller's stream.  No allocation, no synchronisation, no
// global state.
#include <hip/hip_runtime.h>

#include "bole.h"

extern "C" {
int bole_tree_prep_launch(const int32_t*, const int32_t*, int32_t, int32_t, const float*,
                          int32_t, int32_t, int32_t*, uint64_t*, int32_t*, int32_t*, float*,
                          uint32_t*, hipStream_t);
int bole_factor_gc_launch(int32_t, const void*, const void*, const float*, const float*,
                          const uint64_t*, const int32_t*, const int32_t*, int32_t, int32_t,
                          int32_t, int32_t, float*, float*, uint32_t*, hipStream_t);
int bole_verify_launch(int32_t, const void*, const void*, const void*, const float*,
                       const float*, const float*, int32_t, const int32_t*, const float*,
                       const float*, const int32_t*, const int32_t*, const int32_t*,
                       const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                       float*, uint32_t*, hipStream_t);
int bole_verify_neumann_launch(int32_t, const void*, const void*, const void*, const float*,
                               const float*, const float*, int32_t, const int32_t*, const float*,
                               const float*, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                               float*, uint32_t*, hipStream_t);
int bole_verify_inverse_launch(int32_t, const void*, const void*, const void*, const float*,
                               const float*, const float*, int32_t, const int32_t*, const float*,
                               const float*, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                               float*, uint32_t*, hipStream_t);
int bole_factor_inverse_launch(int32_t, const void*, const void*, const float*, const float*,
                               const uint64_t*, const int32_t*, const int32_t*, int32_t, int32_t,
                               int32_t, int32_t, float*, float*, uint32_t*, hipStream_t);
int bole_factor_verify_max_dk(int32_t);
int bole_factor_verify_launch(int32_t, const void*, const void*, const void*, const float*,
                              const float*, const float*, int32_t, const int32_t*,
                              const uint64_t*, const int32_t*, const int32_t*, const int32_t*,
                              const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                              float*, uint32_t*, hipStream_t);
int bole_tree_verify_launch(int32_t, const void*, const void*, const void*, const int32_t*,
                            const float*, const float*, const float*, int32_t, const int32_t*,
                            const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                            float*, int32_t*, uint64_t*, int32_t*, int32_t*, float*, uint32_t*,
                            hipStream_t);
int bole_commit_tree_verify_launch(int32_t, const void*, const void*, const void*, const int32_t*,
                                   const float*, const float*, float*, int32_t, const int32_t*,
                                   const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                   void*, float*, int32_t*, uint64_t*, int32_t*, int32_t*, float*,
                                   const void*, const float*, const float*, const uint64_t*,
                                   const int32_t*, const int32_t*, int32_t, uint32_t*,
                                   hipStream_t);
int bole_tree_conv_launch(int32_t, const void*, const float*, const float*, const void*, int32_t,
                          const int32_t*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t,
                          int32_t, void*, uint32_t*, hipStream_t);
int bole_conv_commit_launch(int32_t, void*, int32_t, const int32_t*, const void*, const int32_t*,
                            const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                            uint32_t*, hipStream_t);
int bole_forest_build_launch(const int32_t*, const float*, const int32_t*, int32_t, int32_t,
                             int32_t, int32_t, float*, int32_t*, int32_t*, int32_t*, void*,
                             uint32_t*, hipStream_t);
int bole_forest_scratch(size_t, void**);
int bole_commit_launch(int32_t, float*, int64_t, int32_t, const int32_t*, int32_t, const void*,
                       int64_t, const float*, int64_t, const float*, int64_t, const uint64_t*,
                       const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                       int32_t, uint32_t*, hipStream_t);
}

namespace {

constexpr int32_t kMaxGrid = 1 << 30;

bool head_dim_ok(int32_t d) { return d >= 16 && d <= 256 && d % 16 == 0; }

constexpr int32_t kMaxConvWidth = 8;

// budget selection: request ids fit the order key's 12-bit field, and the
// listed keys (B * max_tree) stay within one workgroup's reach
constexpr int32_t kMaxForestRequests = 4095;
constexpr int64_t kMaxForestListed = 16384;

bool forest_shape_ok(int32_t B, int32_t max_tree) {
  return B >= 1 && B <= kMaxForestRequests && max_tree >= 1 && max_tree <= BOLE_MAX_TREE &&
         (int64_t)B * max_tree <= kMaxForestListed;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int32_t dt) { return dt == BOLE_F32 || dt == BOLE_BF16; }

// B * H * tiles must fit a 1-D grid
bool grid_ok(int64_t B, int64_t H, int64_t tiles) { return B * H * tiles < kMaxGrid; }

using VerifyLaunch = int (*)(int32_t, const void*, const void*, const void*, const float*,
                             const float*, const float*, int32_t, const int32_t*, const float*,
                             const float*, const int32_t*, const int32_t*, const int32_t*,
                             const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                             float*, uint32_t*, hipStream_t);

// bole_verify and its alternative solves share their argument checks
int verify_checked(VerifyLaunch launch, int32_t dtype, const void* q, const void* k,
                   const void* v, const float* logP, const float* beta, const float* state_pool,
                   int32_t n_slots, const int32_t* slot, const float* G, const float* C,
                   const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                   const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                   int32_t d_v, void* O, float* U, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!q || !k || !v || !logP || !beta || !state_pool || !slot || !G || !C || !order || !depth ||
      !tree_off || !tree_depth || !O || !U)
    return BOLE_E_NULL;
  if (B < 1 || N < 1 || H < 1 || n_slots < 1 || !grid_ok(B, H, 4)) return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return BOLE_E_UNSUPPORTED;
  return launch(dtype, q, k, v, logP, beta, state_pool, n_slots, slot, G, C, order, depth,
                tree_off, tree_depth, B, N, H, d_k, d_v, O, U, err, (hipStream_t)stream);
}

using FactorLaunch = int (*)(int32_t, const void*, const void*, const float*, const float*,
                             const uint64_t*, const int32_t*, const int32_t*, int32_t, int32_t,
                             int32_t, int32_t, float*, float*, uint32_t*, hipStream_t);

int factor_checked(FactorLaunch launch, int32_t dtype, const void* q, const void* k,
                   const float* logP, const float* beta, const uint64_t* anc,
                   const int32_t* order, const int32_t* tree_off, int32_t B, int32_t N,
                   int32_t H, int32_t d_k, float* G, float* C, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!q || !k || !logP || !beta || !anc || !order || !tree_off || !G || !C) return BOLE_E_NULL;
  if (B < 1 || N < 1 || H < 1 || !grid_ok(B, H, 1)) return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k)) return BOLE_E_UNSUPPORTED;
  return launch(dtype, q, k, logP, beta, anc, order, tree_off, B, N, H, d_k, G, C, err,
                (hipStream_t)stream);
}
}  // namespace

extern "C" {

int bole_tree_prep(const int32_t* parent, const int32_t* tree_off, int32_t B, int32_t N,
                   const float* log_gamma, int32_t L, int32_t H, int32_t* depth, uint64_t* anc,
                   int32_t* order, int32_t* tree_depth, float* logP, uint32_t* err,
                   void* stream) {
  if (!parent || !tree_off || !depth || !anc || !order || !tree_depth) return BOLE_E_NULL;
  if (B < 1 || N < 1 || B > (1 << 24)) return BOLE_E_SHAPE;
  if (log_gamma) {
    if (!logP) return BOLE_E_NULL;
    if (L < 1 || H < 1 || (int64_t)L * H > (1 << 24)) return BOLE_E_SHAPE;
  }
  return bole_tree_prep_launch(parent, tree_off, B, N, log_gamma, L, H, depth, anc, order,
                               tree_depth, log_gamma ? logP : nullptr, err,
                               (hipStream_t)stream);
}

size_t bole_gc_workspace_bytes(int32_t B, int32_t H) {
  if (B < 1 || H < 1) return 0;
  return (size_t)2 * B * H * BOLE_MAX_TREE * BOLE_MAX_TREE * sizeof(float);
}

int bole_factor_gc(int32_t dtype, const void* q, const void* k, const float* logP,
                   const float* beta, const uint64_t* anc, const int32_t* order,
                   const int32_t* tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
                   float* G, float* C, uint32_t* err, void* stream) {
  return factor_checked(bole_factor_gc_launch, dtype, q, k, logP, beta, anc, order, tree_off, B,
                        N, H, d_k, G, C, err, stream);
}

int bole_verify(int32_t dtype, const void* q, const void* k, const void* v, const float* logP,
                const float* beta, const float* state_pool, int32_t n_slots, const int32_t* slot,
                const float* G, const float* C, const int32_t* order, const int32_t* depth,
                const int32_t* tree_off, const int32_t* tree_depth, int32_t B, int32_t N,
                int32_t H, int32_t d_k, int32_t d_v, void* O, float* U, uint32_t* err,
                void* stream) {
  return verify_checked(bole_verify_launch, dtype, q, k, v, logP, beta, state_pool, n_slots, slot,
                        G, C, order, depth, tree_off, tree_depth, B, N, H, d_k, d_v, O, U, err,
                        stream);
}

int bole_verify_neumann(int32_t dtype, const void* q, const void* k, const void* v,
                        const float* logP, const float* beta, const float* state_pool,
                        int32_t n_slots, const int32_t* slot, const float* G, const float* C,
                        const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                        const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                        int32_t d_v, void* O, float* U, uint32_t* err, void* stream) {
  return verify_checked(bole_verify_neumann_launch, dtype, q, k, v, logP, beta, state_pool,
                        n_slots, slot, G, C, order, depth, tree_off, tree_depth, B, N, H, d_k,
                        d_v, O, U, err, stream);
}

int bole_verify_inverse(int32_t dtype, const void* q, const void* k, const void* v,
                        const float* logP, const float* beta, const float* state_pool,
                        int32_t n_slots, const int32_t* slot, const float* W, const float* M,
                        const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                        const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                        int32_t d_v, void* O, float* U, uint32_t* err, void* stream) {
  return verify_checked(bole_verify_inverse_launch, dtype, q, k, v, logP, beta, state_pool,
                        n_slots, slot, W, M, order, depth, tree_off, tree_depth, B, N, H, d_k,
                        d_v, O, U, err, stream);
}

int bole_factor_inverse(int32_t dtype, const void* q, const void* k, const float* logP,
                        const float* beta, const uint64_t* anc, const int32_t* order,
                        const int32_t* tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
                        float* W, float* M, uint32_t* err, void* stream) {
  return factor_checked(bole_factor_inverse_launch, dtype, q, k, logP, beta, anc, order, tree_off,
                        B, N, H, d_k, W, M, err, stream);
}

int bole_factor_verify(int32_t dtype, const void* q, const void* k, const void* v,
                       const float* logP, const float* beta, const float* state_pool,
                       int32_t n_slots, const int32_t* slot, const uint64_t* anc,
                       const int32_t* order, const int32_t* depth, const int32_t* tree_off,
                       const int32_t* tree_depth, int32_t B, int32_t N, int32_t H, int32_t d_k,
                       int32_t d_v, void* O, float* U, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!q || !k || !v || !logP || !beta || !state_pool || !slot || !anc || !order || !depth ||
      !tree_off || !tree_depth || !O || !U)
    return BOLE_E_NULL;
  if (B < 1 || N < 1 || H < 1 || n_slots < 1 || !grid_ok(B, H, 4)) return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v) || d_k > bole_factor_verify_max_dk(dtype))
    return BOLE_E_UNSUPPORTED;
  return bole_factor_verify_launch(dtype, q, k, v, logP, beta, state_pool, n_slots, slot, anc,
                                   order, depth, tree_off, tree_depth, B, N, H, d_k, d_v, O, U,
                                   err, (hipStream_t)stream);
}

int bole_tree_verify(int32_t dtype, const void* q, const void* k, const void* v,
                     const int32_t* parent, const float* log_gamma, const float* beta,
                     const float* state_pool, int32_t n_slots, const int32_t* slot,
                     const int32_t* tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
                     int32_t d_v, void* O, float* U, int32_t* depth, uint64_t* anc,
                     int32_t* order, int32_t* tree_depth, float* logP, uint32_t* err,
                     void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!q || !k || !v || !parent || !log_gamma || !beta || !state_pool || !slot || !tree_off ||
      !O || !U || !depth || !anc || !order || !tree_depth || !logP)
    return BOLE_E_NULL;
  if (B < 1 || N < 1 || H < 1 || n_slots < 1 || B > (1 << 24) || !grid_ok(B, H, 4))
    return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v) || d_k > bole_factor_verify_max_dk(dtype))
    return BOLE_E_UNSUPPORTED;
  return bole_tree_verify_launch(dtype, q, k, v, parent, log_gamma, beta, state_pool, n_slots,
                                 slot, tree_off, B, N, H, d_k, d_v, O, U, depth, anc, order,
                                 tree_depth, logP, err, (hipStream_t)stream);
}

int bole_commit_tree_verify(int32_t dtype, const void* q, const void* k, const void* v,
                            const int32_t* parent, const float* log_gamma, const float* beta,
                            float* state_pool, int32_t n_slots, const int32_t* slot,
                            const int32_t* tree_off, int32_t B, int32_t N, int32_t H, int32_t d_k,
                            int32_t d_v, void* O, float* U, int32_t* depth, uint64_t* anc,
                            int32_t* order, int32_t* tree_depth, float* logP, const void* prev_k,
                            const float* prev_U, const float* prev_logP, const uint64_t* prev_anc,
                            const int32_t* prev_tree_off, const int32_t* prev_accept,
                            int32_t prev_N, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!q || !k || !v || !parent || !log_gamma || !beta || !state_pool || !slot || !tree_off ||
      !O || !U || !depth || !anc || !order || !tree_depth || !logP || !prev_k || !prev_U ||
      !prev_logP || !prev_anc || !prev_tree_off || !prev_accept)
    return BOLE_E_NULL;
  if (B < 1 || N < 1 || H < 1 || n_slots < 1 || prev_N < 1 || B > (1 << 24) || !grid_ok(B, H, 4))
    return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v) || d_k > bole_factor_verify_max_dk(dtype) ||
      (uintptr_t)prev_k % 8 != 0)
    return BOLE_E_UNSUPPORTED;
  return bole_commit_tree_verify_launch(
      dtype, q, k, v, parent, log_gamma, beta, state_pool, n_slots, slot, tree_off, B, N, H, d_k,
      d_v, O, U, depth, anc, order, tree_depth, logP, prev_k, prev_U, prev_logP, prev_anc,
      prev_tree_off, prev_accept, prev_N, err, (hipStream_t)stream);
}

int bole_tree_conv(int32_t dtype, const void* x, const float* weight, const float* bias,
                   const void* conv_state, int32_t n_slots, const int32_t* slot,
                   const int32_t* parent, const int32_t* tree_off, int32_t B, int32_t N, int32_t C,
                   int32_t W, void* y, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!x || !weight || !parent || !tree_off || !y || (W > 1 && (!conv_state || !slot)))
    return BOLE_E_NULL;
  if (B < 1 || N < 1 || C < 1 || B > (1 << 24) || (W > 1 && n_slots < 1)) return BOLE_E_SHAPE;
  if (W < 1 || W > kMaxConvWidth || C % 8 != 0 || C > (1 << 24) || !aligned16(x) ||
      !aligned16(y) || (W > 1 && !aligned16(conv_state)))
    return BOLE_E_UNSUPPORTED;
  return bole_tree_conv_launch(dtype, x, weight, bias, conv_state, n_slots, slot, parent,
                               tree_off, B, N, C, W, y, err, (hipStream_t)stream);
}

int bole_conv_commit(int32_t dtype, void* conv_state, int32_t n_slots, const int32_t* slot,
                     const void* x, const int32_t* parent, const int32_t* tree_off,
                     const int32_t* accept, int32_t B, int32_t N, int32_t C, int32_t W,
                     uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if ((W > 1 && !conv_state) || !slot || !x || !parent || !tree_off || !accept) return BOLE_E_NULL;
  if (B < 1 || N < 1 || C < 1 || n_slots < 1 || B > (1 << 24)) return BOLE_E_SHAPE;
  if (W < 1 || W > kMaxConvWidth || C > (1 << 24)) return BOLE_E_UNSUPPORTED;
  if (W == 1) return BOLE_OK;  // no state to move
  return bole_conv_commit_launch(dtype, conv_state, n_slots, slot, x, parent, tree_off, accept, B,
                                 N, C, W, err, (hipStream_t)stream);
}

size_t bole_forest_workspace_bytes(int32_t B, int32_t max_tree) {
  if (!forest_shape_ok(B, max_tree)) return 0;
  return (size_t)12 * B * max_tree;  // a key and a parent position per listed slot
}

int bole_forest_build(const int32_t* cand_parent, const float* p_draft, const int32_t* cand_off,
                      int32_t B, int32_t M_total, int32_t capacity, int32_t max_tree, float* rho,
                      int32_t* parent, int32_t* cand_of, int32_t* tree_off, void* workspace,
                      uint32_t* err, void* stream) {
  if (!cand_parent || !p_draft || !cand_off || !rho || !parent || !cand_of || !tree_off ||
      !workspace)
    return BOLE_E_NULL;
  if (!forest_shape_ok(B, max_tree) || M_total < 1 || capacity < 1) return BOLE_E_SHAPE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return BOLE_E_UNSUPPORTED;
  return bole_forest_build_launch(cand_parent, p_draft, cand_off, B, M_total, capacity, max_tree,
                                  rho, parent, cand_of, tree_off, workspace, err,
                                  (hipStream_t)stream);
}

int bole_forest_build_noalloc(const int32_t* cand_parent, const float* p_draft,
                              const int32_t* cand_off, int32_t B, int32_t M_total,
                              int32_t capacity, int32_t max_tree, float* rho, int32_t* parent,
                              int32_t* cand_of, int32_t* tree_off, uint32_t* err, void* stream) {
  if (!cand_parent || !p_draft || !cand_off || !rho || !parent || !cand_of || !tree_off)
    return BOLE_E_NULL;
  if (!forest_shape_ok(B, max_tree) || M_total < 1 || capacity < 1) return BOLE_E_SHAPE;
  void* scratch = nullptr;
  const int st = bole_forest_scratch(bole_forest_workspace_bytes(B, max_tree), &scratch);
  if (st != BOLE_OK) return st;
  return bole_forest_build_launch(cand_parent, p_draft, cand_off, B, M_total, capacity, max_tree,
                                  rho, parent, cand_of, tree_off, scratch, err,
                                  (hipStream_t)stream);
}

int bole_commit_path(int32_t L, float* state_pool, int64_t state_layer_stride, int32_t n_slots,
                     const int32_t* slot, int32_t dtype, const void* k, int64_t k_layer_stride,
                     const float* U, int64_t u_layer_stride, const float* logP,
                     int64_t logp_layer_stride, const uint64_t* anc, const int32_t* tree_off,
                     const int32_t* accept, int32_t B, int32_t N, int32_t H, int32_t d_k,
                     int32_t d_v, uint32_t* err, void* stream) {
  if (!dtype_ok(dtype)) return BOLE_E_DTYPE;
  if (!state_pool || !slot || !k || !U || !logP || !anc || !tree_off || !accept)
    return BOLE_E_NULL;
  if (L < 1 || L > 65535 || B < 1 || N < 1 || H < 1 || n_slots < 1 || !grid_ok(B, H, 16))
    return BOLE_E_SHAPE;
  if (state_layer_stride < 0 || k_layer_stride < 0 || u_layer_stride < 0 ||
      logp_layer_stride < 0)
    return BOLE_E_SHAPE;
  if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return BOLE_E_UNSUPPORTED;
  return bole_commit_launch(L, state_pool, state_layer_stride, n_slots, slot, dtype, k,
                            k_layer_stride, U, u_layer_stride, logP, logp_layer_stride, anc,
                            tree_off, accept, B, N, H, d_k, d_v, err, (hipStream_t)stream);
}

const char* bole_status_string(int code) {
  switch (code) {
    case BOLE_OK: return "ok";
    case BOLE_E_NULL: return "a required pointer is NULL";
    case BOLE_E_SHAPE: return "a size argument is out of range";
    case BOLE_E_DTYPE: return "unknown element type";
    case BOLE_E_UNSUPPORTED: return "head dimension must be a multiple of 16 in [16, 256]";
    case BOLE_E_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
