// Calibration kernels (not part of the bdmoe ABI): a copy for the HBM
// traffic counters and a read-only stream that measures the box's
// achievable read bandwidth for the weight-streaming access pattern.
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

// bdmcal_stream_read reads `bytes` bytes (a multiple of 16) once: a
// grid-stride loop over 32 KiB chunks (a workgroup reads one contiguous
// chunk per step, a wave 1 KiB per load instruction), every lane keeping
// two batches of 8 non-temporal 16-byte loads in flight (ping-pong) and
// folding them into an XOR (written per thread to `out`, so the loads cannot
// be dropped).
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   long n16,
                                                                   uint32_t* __restrict__ out) {
  constexpr long kBatch = static_cast<long>(kReadThreads) * kReadUnroll;   // 16-byte units
  const long stride = static_cast<long>(gridDim.x) * kBatch;
  long i = static_cast<long>(blockIdx.x) * kBatch + threadIdx.x;
  uint32_t acc = 0u;
  u32x4 a[kReadUnroll], b[kReadUnroll];
  auto full = [&](long base) { return base + (kReadUnroll - 1) * kReadThreads < n16; };
  auto load = [&](long base, u32x4(&v)[kReadUnroll]) {
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + base + u * kReadThreads);
  };
  auto fold = [&](const u32x4(&v)[kReadUnroll]) {
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  };
  if (full(i)) {
    load(i, a);
    for (;;) {
      const bool nb = full(i + stride);
      if (nb) load(i + stride, b);
      fold(a);
      i += stride;
      if (!nb) break;
      const bool na = full(i + stride);
      if (na) load(i + stride, a);
      fold(b);
      i += stride;
      if (!na) break;
    }
  }
  // the rest of a partial chunk (only past the last full one)
  for (; i < n16; i += kReadThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<long>(blockIdx.x) * kReadThreads + threadIdx.x] = acc;
}

// The same read in the other common order: workgroup b reads its own
// contiguous region (bytes / blocks, rounded down to whole 16 KiB batches;
// the remainder is not read), 4 loads per lane per batch, two batches in
// flight.  With one workgroup per CU this is the order of a persistent
// kernel that gives each workgroup one run of weight rows.
constexpr int kRegUnroll = 4;

__global__ __launch_bounds__(kReadThreads) void stream_read_region_kernel(
    const u32x4* __restrict__ src, long per, uint32_t* __restrict__ out) {
  constexpr long kB = static_cast<long>(kReadThreads) * kRegUnroll;     // 16-byte units
  const long begin = static_cast<long>(blockIdx.x) * per;
  const long end = begin + per;
  uint32_t acc = 0u;
  u32x4 a[kRegUnroll], b[kRegUnroll];
  auto load = [&](long base, u32x4(&v)[kRegUnroll]) {
#pragma unroll
    for (int u = 0; u < kRegUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + base + u * kReadThreads + threadIdx.x);
  };
  auto fold = [&](const u32x4(&v)[kRegUnroll]) {
#pragma unroll
    for (int u = 0; u < kRegUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  };
  long i = begin;                                  // batch base, a multiple of kB
  if (i < end) {
    load(i, a);
    for (;;) {
      const bool nb = i + kB < end;
      if (nb) load(i + kB, b);
      fold(a);
      i += kB;
      if (!nb) break;
      const bool na = i + kB < end;
      if (na) load(i + kB, a);
      fold(b);
      i += kB;
      if (!na) break;
    }
  }
  out[static_cast<long>(blockIdx.x) * kReadThreads + threadIdx.x] = acc;
}

}  // namespace bdmcal

extern "C" __attribute__((visibility("default"))) int bdmcal_stream_read_region(
    const void* src, long bytes, uint32_t* out, int blocks, void* stream) {
  using namespace bdmcal;
  // out: blocks * 256 entries; every workgroup gets at least one batch
  constexpr long kB = static_cast<long>(kReadThreads) * kRegUnroll;
  if (!src || !out || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65535) return -1;
  if (reinterpret_cast<uintptr_t>(src) & 15) return -1;
  const long per = (bytes / 16 / blocks) / kB * kB;
  if (per < kB) return -1;
  (void)hipGetLastError();
  stream_read_region_kernel<<<blocks, kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), per, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" __attribute__((visibility("default"))) int bdmcal_stream_read(const void* src,
                                                                        long bytes,
                                                                        uint32_t* out,
                                                                        int blocks,
                                                                        void* stream) {
  using namespace bdmcal;
  // out: blocks * 256 entries
  if (!src || !out || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65535) return -1;
  if (reinterpret_cast<uintptr_t>(src) & 15) return -1;
  (void)hipGetLastError();
  stream_read_kernel<<<blocks, kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

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
