// Calibration copy for HBM traffic counters (not part of the bdmoe ABI).
//
// bdmcal_stream_copy copies `bytes` bytes (a multiple of 16 KiB) with the
// access pattern of the weight-streaming kernels: every lane reads 16 bytes
// with a non-temporal load, a wave reads 1 KB contiguous, and writes them
// back with an ordinary 16-byte store.  Counter readings of one launch
// against its known size give the scale factors of FETCH_SIZE and
// WRITE_SIZE for that kind of request.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdmcal {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 4;
constexpr long kChunk = 16L * kThreads * kPerThread;   // bytes per workgroup

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst) {
  const long base = static_cast<long>(blockIdx.x) * (kThreads * kPerThread) + threadIdx.x;
  u32x4 v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) v[i] = __builtin_nontemporal_load(src + base + i * kThreads);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) dst[base + i * kThreads] = v[i];
}

}  // namespace bdmcal

extern "C" __attribute__((visibility("default"))) int bdmcal_stream_copy(const void* src,
                                                                        void* dst, long bytes,
                                                                        void* stream) {
  using namespace bdmcal;
  if (!src || !dst || bytes <= 0 || bytes % kChunk != 0 || bytes / kChunk > 0x7fffffffL) return -1;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if ((a | b) & 15) return -1;
  if (a < b + bytes && b < a + bytes) return -1;   // overlap
  (void)hipGetLastError();
  stream_copy_kernel<<<static_cast<unsigned>(bytes / kChunk), kThreads, 0,
                       static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src),
                                                           static_cast<u32x4*>(dst));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
