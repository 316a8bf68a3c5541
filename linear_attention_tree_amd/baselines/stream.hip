// A plain streaming kernel: the bandwidth ceiling the verify kernels are set
// against.  One launch reads n_read 16-byte vectors from src and writes
// n_write to dst, both in grid-stride order, so every wave moves whole 128-byte
// lines back to back.  Called with the read and write byte counts of a verify
// launch, over as many rotated buffers as the verify's timing rotates input
// sets, it gives the rate at which the same bytes move with no dependency
// between reading and writing them.  It is a measurement baseline, not part of
// libbole's interface.
//
// The reads are summed and the sum goes into every written vector, so no read
// can be dropped; the writes are non-temporal, as the verify's outputs are.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void stream_mix_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                  int64_t n_read, int64_t n_write) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = tid; i < n_read; i += nt) acc += src[i];
  for (int64_t i = tid; i < n_write; i += nt) {
    f32x4 o = acc;
    o[0] += (float)i;
    __builtin_nontemporal_store(o, dst + i);
  }
}

}  // namespace

#define BASELINE_API extern "C" __attribute__((visibility("default")))

// n_read / n_write: 16-byte vectors read from src / written to dst (both
// 16-byte aligned when their count is positive).  grid: 1 .. 65536
// workgroups; block: a multiple of 64 up to 1024 threads.  Returns 0, 2 for a
// bad size or alignment, 5 for a failed launch.
BASELINE_API int stream_mix(const void* src, void* dst, int64_t n_read, int64_t n_write,
                            int32_t grid, int32_t block, void* stream) {
  if (n_read < 0 || n_write < 0 || grid < 1 || grid > 65536 || block < 64 || block > 1024 ||
      block % 64 != 0)
    return 2;
  if ((n_read > 0 && (src == nullptr || (uintptr_t)src % 16 != 0)) ||
      (n_write > 0 && (dst == nullptr || (uintptr_t)dst % 16 != 0)))
    return 2;
  hipLaunchKernelGGL(stream_mix_kernel, dim3(grid), dim3(block), 0, (hipStream_t)stream,
                     reinterpret_cast<const f32x4*>(src), reinterpret_cast<f32x4*>(dst), n_read,
                     n_write);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
