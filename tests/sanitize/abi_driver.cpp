// The host-side argument layer of libbole (csrc/bole_api.hip) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU.  Test
// infrastructure: built and run by tests/test_sanitizers.py on the CPU.
//
// The layer is compiled here as ordinary host C++ and its kernel launchers are
// replaced by stubs that count their calls and return a sentinel.  Each entry
// point must reject bad arguments with its status code before any launcher
// runs, and pass good arguments to exactly one launcher, returning its result.
#include "bole_api.hip"

#include <cstdio>

namespace {
int calls = 0;
constexpr int kSentinel = 4242;
int failures = 0;

#define CHECK(cond)                                                           \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

// a rejected call returns `code` and launches nothing; an accepted one
// launches once and returns the launcher's result
#define REJECTS(code, call)   \
  do {                        \
    const int c0 = calls;     \
    CHECK((call) == (code));  \
    CHECK(calls == c0);       \
  } while (0)
#define LAUNCHES(call)             \
  do {                             \
    const int c0 = calls;          \
    CHECK((call) == kSentinel);    \
    CHECK(calls == c0 + 1);        \
  } while (0)
}  // namespace

#define STUB return (++calls, kSentinel)
extern "C" {
int bole_tree_prep_launch(const int32_t*, const int32_t*, int32_t, int32_t, const float*, int32_t,
                          int32_t, int32_t*, uint64_t*, int32_t*, int32_t*, float*, uint32_t*,
                          hipStream_t) { STUB; }
int bole_factor_gc_launch(int32_t, const void*, const void*, const float*, const float*,
                          const uint64_t*, const int32_t*, const int32_t*, int32_t, int32_t,
                          int32_t, int32_t, float*, float*, uint32_t*, hipStream_t) { STUB; }
int bole_verify_launch(int32_t, const void*, const void*, const void*, const float*, const float*,
                       const float*, int32_t, const int32_t*, const float*, const float*,
                       const int32_t*, const int32_t*, const int32_t*, const int32_t*, int32_t,
                       int32_t, int32_t, int32_t, int32_t, void*, float*, uint32_t*,
                       hipStream_t) { STUB; }
int bole_verify_neumann_launch(int32_t, const void*, const void*, const void*, const float*,
                               const float*, const float*, int32_t, const int32_t*, const float*,
                               const float*, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                               float*, uint32_t*, hipStream_t) { STUB; }
int bole_verify_inverse_launch(int32_t, const void*, const void*, const void*, const float*,
                               const float*, const float*, int32_t, const int32_t*, const float*,
                               const float*, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                               float*, uint32_t*, hipStream_t) { STUB; }
int bole_factor_inverse_launch(int32_t, const void*, const void*, const float*, const float*,
                               const uint64_t*, const int32_t*, const int32_t*, int32_t, int32_t,
                               int32_t, int32_t, float*, float*, uint32_t*, hipStream_t) { STUB; }
int bole_factor_verify_max_dk(int32_t dtype) { return dtype == BOLE_BF16 ? 128 : 64; }
int bole_factor_verify_launch(int32_t, const void*, const void*, const void*, const float*,
                              const float*, const float*, int32_t, const int32_t*,
                              const uint64_t*, const int32_t*, const int32_t*, const int32_t*,
                              const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                              float*, uint32_t*, hipStream_t) { STUB; }
int bole_tree_verify_launch(int32_t, const void*, const void*, const void*, const int32_t*,
                            const float*, const float*, const float*, int32_t, const int32_t*,
                            const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, void*,
                            float*, int32_t*, uint64_t*, int32_t*, int32_t*, float*, uint32_t*,
                            hipStream_t) { STUB; }
int bole_commit_tree_verify_launch(int32_t, const void*, const void*, const void*, const int32_t*,
                                   const float*, const float*, float*, int32_t, const int32_t*,
                                   const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                   void*, float*, int32_t*, uint64_t*, int32_t*, int32_t*, float*,
                                   const void*, const float*, const float*, const uint64_t*,
                                   const int32_t*, const int32_t*, int32_t, uint32_t*,
                                   hipStream_t) { STUB; }
int bole_tree_conv_launch(int32_t, const void*, const float*, const float*, const void*, int32_t,
                          const int32_t*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t,
                          int32_t, void*, uint32_t*, hipStream_t) { STUB; }
int bole_conv_commit_launch(int32_t, void*, int32_t, const int32_t*, const void*, const int32_t*,
                            const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                            uint32_t*, hipStream_t) { STUB; }
int bole_forest_build_launch(const int32_t*, const float*, const int32_t*, int32_t, int32_t,
                             int32_t, int32_t, float*, int32_t*, int32_t*, int32_t*, void*,
                             uint32_t*, hipStream_t) { STUB; }
int bole_commit_launch(int32_t, float*, int64_t, int32_t, const int32_t*, int32_t, const void*,
                       int64_t, const float*, int64_t, const float*, int64_t, const uint64_t*,
                       const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                       int32_t, uint32_t*, hipStream_t) { STUB; }
// the allocation-free builder's scratch lookup: a fixed host buffer here
alignas(256) static unsigned char fake_scratch[12 * 16384];
int bole_forest_scratch(size_t bytes, void** out) {
  if (bytes > sizeof(fake_scratch)) return BOLE_E_SHAPE;
  *out = fake_scratch;
  return BOLE_OK;
}
}

int main() {
  // host buffers stand in for device pointers: the layer never dereferences them
  alignas(16) static char buf[4096];
  void* p = buf;
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  int32_t* iw = reinterpret_cast<int32_t*>(buf);
  const float* fp = reinterpret_cast<const float*>(buf);
  float* fw = reinterpret_cast<float*>(buf);
  const uint64_t* up = reinterpret_cast<const uint64_t*>(buf);
  uint64_t* uw = reinterpret_cast<uint64_t*>(buf);
  uint32_t* err = reinterpret_cast<uint32_t*>(buf);
  void* odd = buf + 4;  // not 8- or 16-byte aligned

  // tree preparation
  LAUNCHES(bole_tree_prep(ip, ip, 16, 1024, fp, 36, 32, iw, uw, iw, iw, fw, err, nullptr));
  LAUNCHES(bole_tree_prep(ip, ip, 1, 1, nullptr, 0, 0, iw, uw, iw, iw, nullptr, nullptr, nullptr));
  REJECTS(BOLE_E_NULL, bole_tree_prep(nullptr, ip, 1, 1, nullptr, 0, 0, iw, uw, iw, iw, nullptr,
                                      err, nullptr));
  REJECTS(BOLE_E_NULL, bole_tree_prep(ip, ip, 1, 1, fp, 1, 1, iw, uw, iw, iw, nullptr, err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_tree_prep(ip, ip, 0, 1, nullptr, 0, 0, iw, uw, iw, iw, nullptr, err,
                                       nullptr));
  REJECTS(BOLE_E_SHAPE, bole_tree_prep(ip, ip, 1, 1, fp, 1 << 13, 1 << 13, iw, uw, iw, iw, fw, err,
                                       nullptr));

  // factors, verify and the alternative solves
  for (auto f : {bole_factor_gc, bole_factor_inverse}) {
    LAUNCHES(f(BOLE_BF16, p, p, fp, fp, up, ip, ip, 16, 1024, 32, 128, fw, fw, err, nullptr));
    REJECTS(BOLE_E_DTYPE, f(9, p, p, fp, fp, up, ip, ip, 16, 1024, 32, 128, fw, fw, err, nullptr));
    REJECTS(BOLE_E_NULL, f(BOLE_F32, p, nullptr, fp, fp, up, ip, ip, 1, 1, 1, 16, fw, fw, err,
                           nullptr));
    REJECTS(BOLE_E_SHAPE, f(BOLE_F32, p, p, fp, fp, up, ip, ip, 1, 1, 0, 16, fw, fw, err, nullptr));
    REJECTS(BOLE_E_SHAPE, f(BOLE_F32, p, p, fp, fp, up, ip, ip, 1 << 16, 1, 1 << 15, 16, fw, fw,
                            err, nullptr));
    REJECTS(BOLE_E_UNSUPPORTED, f(BOLE_F32, p, p, fp, fp, up, ip, ip, 1, 1, 1, 24, fw, fw, err,
                                  nullptr));
    REJECTS(BOLE_E_UNSUPPORTED, f(BOLE_F32, p, p, fp, fp, up, ip, ip, 1, 1, 1, 272, fw, fw, err,
                                  nullptr));
  }
  for (auto f : {bole_verify, bole_verify_neumann, bole_verify_inverse}) {
    LAUNCHES(f(BOLE_BF16, p, p, p, fp, fp, fp, 16, ip, fp, fp, ip, ip, ip, ip, 16, 1024, 32, 128,
               128, p, fw, err, nullptr));
    REJECTS(BOLE_E_DTYPE, f(2, p, p, p, fp, fp, fp, 16, ip, fp, fp, ip, ip, ip, ip, 1, 1, 1, 16,
                            16, p, fw, err, nullptr));
    REJECTS(BOLE_E_NULL, f(BOLE_F32, p, p, p, fp, fp, fp, 1, ip, nullptr, fp, ip, ip, ip, ip, 1, 1,
                           1, 16, 16, p, fw, err, nullptr));
    REJECTS(BOLE_E_SHAPE, f(BOLE_F32, p, p, p, fp, fp, fp, 0, ip, fp, fp, ip, ip, ip, ip, 1, 1, 1,
                            16, 16, p, fw, err, nullptr));
    REJECTS(BOLE_E_UNSUPPORTED, f(BOLE_F32, p, p, p, fp, fp, fp, 1, ip, fp, fp, ip, ip, ip, ip, 1,
                                  1, 1, 16, 8, p, fw, err, nullptr));
  }
  LAUNCHES(bole_factor_verify(BOLE_BF16, p, p, p, fp, fp, fp, 16, ip, up, ip, ip, ip, ip, 16, 1024,
                              32, 128, 128, p, fw, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_factor_verify(BOLE_F32, p, p, p, fp, fp, fp, 16, ip, up, ip, ip,
                                                 ip, ip, 1, 64, 1, 128, 16, p, fw, err, nullptr));
  REJECTS(BOLE_E_NULL, bole_factor_verify(BOLE_F32, p, p, p, fp, fp, fp, 16, ip, nullptr, ip, ip,
                                          ip, ip, 1, 64, 1, 64, 16, p, fw, err, nullptr));

  // preparation inside verify, and the previous round's commit inside it
  LAUNCHES(bole_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fp, 16, ip, ip, 16, 1024, 32, 128, 128,
                            p, fw, iw, uw, iw, iw, fw, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fp, 16, ip, ip, 16,
                                               1024, 32, 256, 128, p, fw, iw, uw, iw, iw, fw, err,
                                               nullptr));
  REJECTS(BOLE_E_NULL, bole_tree_verify(BOLE_BF16, p, p, p, ip, nullptr, fp, fp, 16, ip, ip, 16,
                                        1024, 32, 128, 128, p, fw, iw, uw, iw, iw, fw, err,
                                        nullptr));
  LAUNCHES(bole_commit_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fw, 16, ip, ip, 16, 1024, 32,
                                   128, 128, p, fw, iw, uw, iw, iw, fw, p, fp, fp, up, ip, ip,
                                   1024, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_commit_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fw, 16, ip,
                                                      ip, 16, 1024, 32, 128, 128, p, fw, iw, uw,
                                                      iw, iw, fw, odd, fp, fp, up, ip, ip, 1024,
                                                      err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_commit_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fw, 16, ip, ip, 16,
                                                1024, 32, 128, 128, p, fw, iw, uw, iw, iw, fw, p,
                                                fp, fp, up, ip, ip, 0, err, nullptr));
  REJECTS(BOLE_E_NULL, bole_commit_tree_verify(BOLE_BF16, p, p, p, ip, fp, fp, fw, 16, ip, ip, 16,
                                               1024, 32, 128, 128, p, fw, iw, uw, iw, iw, fw, p,
                                               fp, fp, up, ip, nullptr, 1024, err, nullptr));

  // the tree convolution and its state commit
  LAUNCHES(bole_tree_conv(BOLE_BF16, p, fp, nullptr, p, 16, ip, ip, ip, 16, 1024, 12288, 4, p, err,
                          nullptr));
  LAUNCHES(bole_tree_conv(BOLE_F32, p, fp, fp, nullptr, 0, nullptr, ip, ip, 1, 8, 64, 1, p, err,
                          nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_tree_conv(BOLE_BF16, odd, fp, nullptr, p, 16, ip, ip, ip, 16,
                                             1024, 12288, 4, p, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_tree_conv(BOLE_BF16, p, fp, nullptr, p, 16, ip, ip, ip, 16,
                                             1024, 12290, 4, p, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_tree_conv(BOLE_BF16, p, fp, nullptr, p, 16, ip, ip, ip, 16,
                                             1024, 12288, 9, p, err, nullptr));
  REJECTS(BOLE_E_NULL, bole_tree_conv(BOLE_BF16, p, fp, nullptr, nullptr, 16, ip, ip, ip, 16,
                                      1024, 12288, 4, p, err, nullptr));
  LAUNCHES(bole_conv_commit(BOLE_BF16, p, 16, ip, p, ip, ip, ip, 16, 1024, 12288, 4, err, nullptr));
  REJECTS(BOLE_OK, bole_conv_commit(BOLE_BF16, nullptr, 16, ip, p, ip, ip, ip, 16, 1024, 12288, 1,
                                    err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_conv_commit(BOLE_BF16, p, 0, ip, p, ip, ip, ip, 16, 1024, 12288, 4,
                                         err, nullptr));

  // budget selection and packing
  CHECK(bole_forest_workspace_bytes(16, 64) == 12u * 16 * 64);
  CHECK(bole_forest_workspace_bytes(4096, 1) == 0);
  CHECK(bole_forest_workspace_bytes(300, 64) == 0);
  LAUNCHES(bole_forest_build(ip, fp, ip, 16, 1872, 1024, 64, fw, iw, iw, iw, p, err, nullptr));
  REJECTS(BOLE_E_UNSUPPORTED, bole_forest_build(ip, fp, ip, 16, 1872, 1024, 64, fw, iw, iw, iw,
                                                odd, err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_forest_build(ip, fp, ip, 16, 1872, 0, 64, fw, iw, iw, iw, p, err,
                                          nullptr));
  REJECTS(BOLE_E_SHAPE, bole_forest_build(ip, fp, ip, 16, 1872, 1024, 65, fw, iw, iw, iw, p, err,
                                          nullptr));
  REJECTS(BOLE_E_NULL, bole_forest_build(ip, fp, ip, 16, 1872, 1024, 64, fw, iw, iw, iw, nullptr,
                                         err, nullptr));

  // the allocation-free builder: the same checks, no workspace argument
  LAUNCHES(bole_forest_build_noalloc(ip, fp, ip, 16, 1872, 1024, 64, fw, iw, iw, iw, err, nullptr));
  LAUNCHES(bole_forest_build_noalloc(ip, fp, ip, 256, 20000, 16384, 64, fw, iw, iw, iw, err,
                                     nullptr));
  REJECTS(BOLE_E_SHAPE, bole_forest_build_noalloc(ip, fp, ip, 257, 20000, 16384, 64, fw, iw, iw,
                                                  iw, err, nullptr));
  REJECTS(BOLE_E_NULL, bole_forest_build_noalloc(ip, fp, nullptr, 16, 1872, 1024, 64, fw, iw, iw,
                                                 iw, err, nullptr));

  // the multi-layer commit
  LAUNCHES(bole_commit_path(36, fw, 1 << 20, 32, ip, BOLE_BF16, p, 1 << 20, fp, 1 << 20, fp,
                            1 << 16, up, ip, ip, 32, 2048, 32, 128, 128, err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_commit_path(65536, fw, 0, 32, ip, BOLE_BF16, p, 0, fp, 0, fp, 0, up,
                                         ip, ip, 32, 2048, 32, 128, 128, err, nullptr));
  REJECTS(BOLE_E_SHAPE, bole_commit_path(2, fw, -1, 32, ip, BOLE_BF16, p, 0, fp, 0, fp, 0, up, ip,
                                         ip, 32, 2048, 32, 128, 128, err, nullptr));
  REJECTS(BOLE_E_NULL, bole_commit_path(2, fw, 0, 32, ip, BOLE_BF16, p, 0, fp, 0, fp, 0, up, ip,
                                        nullptr, 32, 2048, 32, 128, 128, err, nullptr));

  // helpers
  CHECK(bole_gc_workspace_bytes(16, 32) == 2u * 16 * 32 * 64 * 64 * 4);
  CHECK(bole_gc_workspace_bytes(-1, 32) == 0);
  for (int code = -2; code < 8; ++code) CHECK(bole_status_string(code) != nullptr);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("ABI sanitizer driver: ok (%d launches)\n", calls);
  return 0;
}
