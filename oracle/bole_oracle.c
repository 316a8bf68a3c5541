/*
 * CPU oracle for closed-form tree verification of Gated DeltaNet layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes is the plain definition the pages give for tree
 * verification: every proposal node's output is the output of ordinary
 * sequential GDN decoding along that node's root-to-node path, started from the
 * immutable pre-tree state (Bole, arXiv 2608.01651, Theorem 1 states that the
 * closed form equals sequential tree execution; the recurrence is Eq. 1 as
 * printed in the xllm-io paper review, section 三 "Gated DeltaNet 递归核心").
 * All state arithmetic is float64.  Build with -ffp-contract=off so that the
 * tree walk and the token-order loop perform identical operation sequences.
 *
 * State layout follows the serving slot layout the pages describe ([H, d_v, d_k]
 * per request, arXiv page, state-lifecycle paragraph): element (v, c) of a slot
 * is S[c][v] of the paper's S in R^{d_k x d_v}.
 *
 * Recurrence (Eq. 1), per token t and head:
 *     S~ = gamma_t S_{t-1};   u_t = beta_t (v_t - S~^T k_t);
 *     S_t = S~ + k_t u_t^T;   o_t = S_t^T q_t,
 * with gamma_t = exp(g_t), g_t the log-gate input.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_MAX_TREE 64

enum {
  REF_ERR_BAD_PARENT = 1,
  REF_ERR_CYCLE = 2,
  REF_ERR_TREE_SIZE = 4,
  REF_ERR_BAD_ACCEPT = 8,
  REF_ERR_BAD_SLOT = 16
};

/* ------------------------------------------------------------------------ */
/* Tree preparation: depth, ancestor-or-self bits, level order, tree depth and
 * the log-space gate products logP_i = sum of g over the root-to-i path,
 * i included (the gate product P_i of Lemma 1 includes gamma_i; review, Eq. 4
 * paragraph).  logP is summed in float32, root first, one rounding per add,
 * starting from +0.0f.  Returns the OR of error bits. */
uint32_t bole_ref_tree_prep(const int32_t* parent, const int32_t* tree_off, int32_t B,
                            int32_t N, const float* log_gamma, int32_t L, int32_t H,
                            int32_t* depth, uint64_t* anc, int32_t* order,
                            int32_t* tree_depth, float* logP) {
  uint32_t err = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t off = tree_off[b], end = tree_off[b + 1];
    int32_t T = end - off;
    if (off < 0 || end > N || T < 1 || T > REF_MAX_TREE) {
      err |= REF_ERR_TREE_SIZE;
      continue;
    }
    int bad = 0;
    for (int32_t i = 0; i < T; ++i) {
      int32_t p = parent[off + i];
      if (p != -1 && (p < 0 || p >= T || p == i)) bad = 1;
    }
    if (bad) {
      err |= REF_ERR_BAD_PARENT;
      continue;
    }
    int cyc = 0;
    int32_t dep[REF_MAX_TREE];
    uint64_t bits[REF_MAX_TREE];
    for (int32_t i = 0; i < T && !cyc; ++i) {
      int32_t x = i, steps = 0;
      uint64_t m = 1ull << i;
      while (parent[off + x] != -1) {
        x = parent[off + x];
        m |= 1ull << x;
        if (++steps > T - 1) {
          cyc = 1;
          break;
        }
      }
      dep[i] = steps;
      bits[i] = m;
    }
    if (cyc) {
      err |= REF_ERR_CYCLE;
      continue;
    }
    int32_t dmax = 0;
    for (int32_t i = 0; i < T; ++i) {
      depth[off + i] = dep[i];
      anc[off + i] = bits[i];
      if (dep[i] > dmax) dmax = dep[i];
    }
    tree_depth[b] = dmax;
    /* stable order by (depth, local index) */
    int32_t pos = 0;
    for (int32_t lev = 0; lev <= dmax; ++lev)
      for (int32_t i = 0; i < T; ++i)
        if (dep[i] == lev) order[off + pos++] = i;
    if (log_gamma && logP) {
      for (int32_t i = 0; i < T; ++i) {
        int32_t path[REF_MAX_TREE];
        int32_t n = 0, x = i;
        for (;;) {
          path[n++] = x;
          if (parent[off + x] == -1) break;
          x = parent[off + x];
        }
        for (int32_t l = 0; l < L; ++l)
          for (int32_t h = 0; h < H; ++h) {
            volatile float acc = 0.0f;
            for (int32_t r = n - 1; r >= 0; --r)
              acc = acc + log_gamma[((int64_t)l * N + off + path[r]) * H + h];
            logP[((int64_t)l * N + off + i) * H + h] = acc;
          }
      }
    }
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* One Eq. 1 step on a [dv][dk] state; writes u (length dv). */
static void gdn_step(double* S, int dk, int dv, const double* k, const double* v, double g,
                     double beta, double* u) {
  const double gamma = exp(g);
  for (int a = 0; a < dv * dk; ++a) S[a] *= gamma;
  for (int j = 0; j < dv; ++j) {
    double w = 0.0;
    for (int c = 0; c < dk; ++c) w += S[j * dk + c] * k[c];
    u[j] = beta * (v[j] - w);
  }
  for (int j = 0; j < dv; ++j)
    for (int c = 0; c < dk; ++c) S[j * dk + c] += u[j] * k[c];
}

static void readout(const double* S, int dk, int dv, const double* q, double* o) {
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int c = 0; c < dk; ++c) acc += S[j * dk + c] * q[c];
    o[j] = acc;
  }
}

/* Ordinary token-order decoding: n tokens, state updated in place.
 * q,k: [n][dk]; v: [n][dv]; o,u: [n][dv] (either may be NULL). */
void bole_ref_sequential(int32_t n, int32_t dk, int32_t dv, double* S, const double* q,
                         const double* k, const double* v, const double* g,
                         const double* beta, double* o, double* u) {
  double* ut = (double*)malloc(sizeof(double) * dv);
  for (int32_t t = 0; t < n; ++t) {
    gdn_step(S, dk, dv, k + (int64_t)t * dk, v + (int64_t)t * dv, g[t], beta[t], ut);
    if (u) memcpy(u + (int64_t)t * dv, ut, sizeof(double) * dv);
    if (o) readout(S, dk, dv, q + (int64_t)t * dk, o + (int64_t)t * dv);
  }
  free(ut);
}

/* ------------------------------------------------------------------------ */
/* thread pool over independent work units */
typedef void (*unit_fn)(void* ctx, int64_t unit);
typedef struct {
  unit_fn fn;
  void* ctx;
  int64_t n;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t u = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (u >= p->n) break;
    p->fn(p->ctx, u);
  }
  return NULL;
}

static void run_pool(unit_fn fn, void* ctx, int64_t n, int nthreads) {
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n = n;
  p.next = 0;
  pthread_mutex_init(&p.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
  pool_worker(&p);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&p.mu);
}

/* Committed prefix states: units independent chains of n tokens from S = 0.
 * Token arrays are [units][n][d]; S_out is [units][dv][dk]. */
typedef struct {
  int32_t n, dk, dv;
  const double *q, *k, *v, *g, *beta;
  double* S;
} prefix_ctx;

static void prefix_unit(void* c, int64_t u) {
  prefix_ctx* x = (prefix_ctx*)c;
  double* S = x->S + u * x->dv * x->dk;
  memset(S, 0, sizeof(double) * x->dv * x->dk);
  bole_ref_sequential(x->n, x->dk, x->dv, S, NULL, x->k + u * x->n * x->dk,
                      x->v + u * x->n * x->dv, x->g + u * x->n, x->beta + u * x->n, NULL, NULL);
}

void bole_ref_prefix_batch(int32_t units, int32_t n, int32_t dk, int32_t dv, const double* q,
                           const double* k, const double* v, const double* g,
                           const double* beta, double* S_out, int32_t nthreads) {
  prefix_ctx c = {n, dk, dv, q, k, v, g, beta, S_out};
  run_pool(prefix_unit, &c, units, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Tree verification by walking every node's parent chain.
 * units (optional, n_units entries) restricts the work to listed (b*H + h)
 * units; outputs of other units are left untouched.
 * q,k: [N][H][dk]; v: [N][H][dv]; g,beta: [N][H]; S_pre: [n_slots][H][dv][dk];
 * slot: [B]; parent: [N] local; tree_off: [B+1].
 * Outputs O, U: [N][H][dv].  If accept != NULL, S_new [B][H][dv][dk] receives
 * the state after the accepted node (or S_pre when accept[b] == -1).
 * Trees are assumed valid (run bole_ref_tree_prep first). */
typedef struct {
  const double *q, *k, *v, *g, *beta, *S_pre;
  const int32_t *slot, *parent, *tree_off, *accept;
  int32_t B, N, H, dk, dv;
  double *O, *U, *S_new;
  const int64_t* units;
} walk_ctx;

static int path_to(const int32_t* parent, int32_t off, int32_t i, int32_t* path) {
  int32_t rev[REF_MAX_TREE];
  int n = 0, x = i;
  for (;;) {
    rev[n++] = x;
    if (parent[off + x] == -1) break;
    x = parent[off + x];
  }
  for (int r = 0; r < n; ++r) path[r] = rev[n - 1 - r];
  return n;
}

static void walk_unit(void* c, int64_t idx) {
  walk_ctx* x = (walk_ctx*)c;
  const int64_t unit = x->units ? x->units[idx] : idx;
  const int32_t b = (int32_t)(unit / x->H), h = (int32_t)(unit % x->H);
  const int32_t dk = x->dk, dv = x->dv, H = x->H;
  const int32_t off = x->tree_off[b], T = x->tree_off[b + 1] - off;
  const double* S0 = x->S_pre + ((int64_t)x->slot[b] * H + h) * dv * dk;
  double* S = (double*)malloc(sizeof(double) * dv * dk);
  double* u = (double*)malloc(sizeof(double) * dv);
  int32_t path[REF_MAX_TREE];
  for (int32_t i = 0; i < T; ++i) {
    int n = path_to(x->parent, off, i, path);
    memcpy(S, S0, sizeof(double) * dv * dk);
    for (int r = 0; r < n; ++r) {
      const int64_t tok = (int64_t)(off + path[r]) * H + h;
      gdn_step(S, dk, dv, x->k + tok * dk, x->v + tok * dv, x->g[tok], x->beta[tok], u);
    }
    const int64_t me = (int64_t)(off + i) * H + h;
    if (x->O) readout(S, dk, dv, x->q + me * dk, x->O + me * dv);
    if (x->U) memcpy(x->U + me * dv, u, sizeof(double) * dv);
  }
  if (x->S_new) {
    double* dst = x->S_new + ((int64_t)b * H + h) * dv * dk;
    const int32_t a = x->accept[b];
    memcpy(dst, S0, sizeof(double) * dv * dk);
    if (a >= 0) {
      int n = path_to(x->parent, off, a, path);
      for (int r = 0; r < n; ++r) {
        const int64_t tok = (int64_t)(off + path[r]) * H + h;
        gdn_step(dst, dk, dv, x->k + tok * dk, x->v + tok * dv, x->g[tok], x->beta[tok], u);
      }
    }
  }
  free(S);
  free(u);
}

void bole_ref_verify(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* S_pre, const int32_t* slot,
                     const int32_t* parent, const int32_t* tree_off, const int32_t* accept,
                     int32_t B, int32_t N, int32_t H, int32_t dk, int32_t dv, double* O,
                     double* U, double* S_new, const int64_t* units, int64_t n_units,
                     int32_t nthreads) {
  walk_ctx c = {q, k, v, g, beta, S_pre, slot, parent, tree_off, accept,
                B, N, H, dk, dv, O, U, S_new, units};
  run_pool(walk_unit, &c, units ? n_units : (int64_t)B * H, nthreads);
}
