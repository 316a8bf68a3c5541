/*
 * The C oracle (oracle/bole_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer, and in a separate build under ThreadSanitizer.
 * Test infrastructure: built and run by tests/test_sanitizers.py on the CPU.
 *
 * Every entry point runs on valid forests (one root, several roots, a 64-node
 * chain, ragged sizes, a one-node tree), tree preparation on each invalid
 * topology it reports (parent out of range, a node its own parent, a cycle,
 * an empty or oversized tree, a range past N), and the thread pool with more
 * threads than units and with a unit list.  A wrong result exits non-zero;
 * the sanitizers abort on a memory error, undefined behaviour or a race.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint32_t bole_ref_tree_prep(const int32_t* parent, const int32_t* tree_off, int32_t B,
                            int32_t N, const float* log_gamma, int32_t L, int32_t H,
                            int32_t* depth, uint64_t* anc, int32_t* order,
                            int32_t* tree_depth, float* logP);
void bole_ref_sequential(int32_t n, int32_t dk, int32_t dv, double* S, const double* q,
                         const double* k, const double* v, const double* g,
                         const double* beta, double* o, double* u);
void bole_ref_prefix_batch(int32_t units, int32_t n, int32_t dk, int32_t dv, const double* q,
                           const double* k, const double* v, const double* g,
                           const double* beta, double* S_out, int32_t nthreads);
void bole_ref_verify(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* S_pre, const int32_t* slot,
                     const int32_t* parent, const int32_t* tree_off, const int32_t* accept,
                     int32_t B, int32_t N, int32_t H, int32_t dk, int32_t dv, double* O,
                     double* U, double* S_new, const int64_t* units, int64_t n_units,
                     int32_t nthreads);

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) { /* xorshift64*, a test-only generator */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static double normal(void) { /* Box-Muller */
  const double u1 = uniform01() + 1e-300, u2 = uniform01();
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}
static double* randn(int64_t n, double scale) {
  double* x = (double*)malloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) x[i] = scale * normal();
  return x;
}

static uint32_t prep(const int32_t* parent, const int32_t* off, int B, int N) {
  int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  uint64_t* anc = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)N);
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* td = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  const int L = 2, H = 3;
  float* g = (float*)malloc(sizeof(float) * (size_t)(L * N * H));
  float* logP = (float*)malloc(sizeof(float) * (size_t)(L * N * H));
  for (int i = 0; i < L * N * H; ++i) g[i] = (float)(-uniform01());
  const uint32_t err = bole_ref_tree_prep(parent, off, B, N, g, L, H, depth, anc, order, td, logP);
  free(depth); free(anc); free(order); free(td); free(g); free(logP);
  return err;
}

/* one layer of the walk over a forest, every unit, all threads variants */
static void walk(const int32_t* parent, const int32_t* off, int B, int H, int dk, int dv,
                 int nthreads, int with_units) {
  const int N = off[B];
  const int n_slots = B + 2;
  double *q = randn((int64_t)N * H * dk, 0.1), *k = randn((int64_t)N * H * dk, 0.1);
  double *v = randn((int64_t)N * H * dv, 1.0), *g = randn((int64_t)N * H, 0.1);
  double* beta = randn((int64_t)N * H, 0.2);
  for (int i = 0; i < N * H; ++i) {
    g[i] = -fabs(g[i]);
    beta[i] = 0.5 + 0.4 * tanh(beta[i]);
  }
  double* S = randn((int64_t)n_slots * H * dv * dk, 0.05);
  int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* accept = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  for (int b = 0; b < B; ++b) {
    slot[b] = n_slots - 1 - b;
    const int T = off[b + 1] - off[b];
    accept[b] = b % 3 == 2 ? -1 : (int32_t)(uniform01() * T);
  }
  double* O = (double*)calloc((size_t)N * H * dv, sizeof(double));
  double* U = (double*)calloc((size_t)N * H * dv, sizeof(double));
  double* Sn = (double*)calloc((size_t)B * H * dv * dk, sizeof(double));
  int64_t* units = NULL;
  int64_t n_units = 0;
  if (with_units) {
    units = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B * H));
    for (int u = 0; u < B * H; u += 2) units[n_units++] = u;
  }
  bole_ref_verify(q, k, v, g, beta, S, slot, parent, off, accept, B, N, H, dk, dv, O, U, Sn,
                  units, n_units, nthreads);
  for (int64_t i = 0; i < (int64_t)N * H * dv; ++i) CHECK(isfinite(O[i]) && isfinite(U[i]));
  /* accept = -1 leaves the state as it was */
  for (int b = 2; b < B; b += 3) {
    if (with_units) break;
    for (int h = 0; h < H; ++h)
      CHECK(memcmp(Sn + ((int64_t)b * H + h) * dv * dk,
                   S + ((int64_t)slot[b] * H + h) * dv * dk, sizeof(double) * dv * dk) == 0);
  }
  free(q); free(k); free(v); free(g); free(beta); free(S); free(slot); free(accept);
  free(O); free(U); free(Sn); free(units);
}

int main(void) {
  /* valid forests */
  {
    const int32_t parent[] = {-1, 0, 0, 1, 1, 2, 2, /* heap-ordered binary tree */
                              -1, -1, 1, 0, 3,     /* two roots, labels not parent-first */
                              -1};                 /* one node */
    const int32_t off[] = {0, 7, 12, 13};
    CHECK(prep(parent, off, 3, 13) == 0);
    walk(parent, off, 3, 2, 16, 32, 4, 0);
    walk(parent, off, 3, 2, 32, 16, 64, 1); /* more threads than units, and a unit list */
  }
  {
    int32_t parent[64 + 40];
    for (int i = 0; i < 64; ++i) parent[i] = i - 1; /* a 64-node chain */
    for (int i = 0; i < 40; ++i)                    /* a random recursive tree */
      parent[64 + i] = i == 0 ? -1 : (int32_t)(uniform01() * i);
    const int32_t off[] = {0, 64, 104};
    CHECK(prep(parent, off, 2, 104) == 0);
    walk(parent, off, 2, 3, 16, 16, 3, 0);
  }
  /* invalid topologies: each reported, nothing written out of range */
  {
    const int32_t bad_parent[] = {-1, 5, 0};
    const int32_t off3[] = {0, 3};
    CHECK(prep(bad_parent, off3, 1, 3) & 1u);
    const int32_t self_parent[] = {-1, 1, 0};
    CHECK(prep(self_parent, off3, 1, 3) & 1u);
    const int32_t cycle[] = {-1, 2, 1};
    CHECK(prep(cycle, off3, 1, 3) & 2u);
    const int32_t empty_off[] = {0, 0, 3};
    const int32_t ok3[] = {-1, 0, 1};
    CHECK(prep(ok3, empty_off, 2, 3) & 4u);
    const int32_t past_off[] = {0, 5};
    CHECK(prep(ok3, past_off, 1, 3) & 4u);
    int32_t big[65];
    for (int i = 0; i < 65; ++i) big[i] = i - 1;
    const int32_t big_off[] = {0, 65};
    CHECK(prep(big, big_off, 1, 65) & 4u);
  }
  /* token-order decoding and the batched prefix states agree bit for bit */
  {
    const int n = 40, dk = 16, dv = 8, units = 5;
    double *q = randn((int64_t)units * n * dk, 0.2), *k = randn((int64_t)units * n * dk, 0.2);
    double *v = randn((int64_t)units * n * dv, 1.0), *g = randn((int64_t)units * n, 0.1);
    double* beta = randn((int64_t)units * n, 0.1);
    for (int i = 0; i < units * n; ++i) {
      g[i] = -fabs(g[i]);
      beta[i] = 0.5 + beta[i];
    }
    double* S_batch = (double*)calloc((size_t)units * dv * dk, sizeof(double));
    bole_ref_prefix_batch(units, n, dk, dv, q, k, v, g, beta, S_batch, 8);
    for (int u = 0; u < units; ++u) {
      double* S = (double*)calloc((size_t)dv * dk, sizeof(double));
      double* o = (double*)malloc(sizeof(double) * (size_t)(n * dv));
      bole_ref_sequential(n, dk, dv, S, q + (int64_t)u * n * dk, k + (int64_t)u * n * dk,
                          v + (int64_t)u * n * dv, g + (int64_t)u * n, beta + (int64_t)u * n, o,
                          NULL);
      CHECK(memcmp(S, S_batch + (int64_t)u * dv * dk, sizeof(double) * dv * dk) == 0);
      free(S);
      free(o);
    }
    free(q); free(k); free(v); free(g); free(beta); free(S_batch);
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
