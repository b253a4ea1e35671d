// Device helpers shared by the gfx950 kernels of libbdmoe.
//
// MFMA used throughout: v_mfma_f32_16x16x32_bf16 (one wave64 computes a
// 16x16 fp32 tile from a 16x32 bf16 A tile and a 32x16 bf16 B tile).
// Register layout, lane l = 16*g + c (c = l % 16, g = l / 16):
//   A operand  (8 x bf16 per lane): row c,    k = 8*g + 0..7
//   B operand  (8 x bf16 per lane): column c, k = 8*g + 0..7
//   C/D        (4 x fp32 per lane): column c, rows 4*g + 0..3
// The kernels only rely on A and B using the same k <-> (g, item) map, so a
// lane's 8 consecutive k values are one 16-byte load from a row-major
// (k-contiguous) operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16-byte loads.  `ld16_stream` marks data read exactly once (expert and head
// weights) as non-temporal so it does not evict reused data from the caches.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Online-softmax statistics of a set of logits: running max m, sum of
// exp(l - m), and the lowest index attaining m (INT32_MAX when empty).
struct SoftStat {
  float m;
  float s;
  int a;
};

__device__ __forceinline__ SoftStat softstat_empty() { return {-INFINITY, 0.0f, INT32_MAX}; }

// Associative merge; the winner is the larger max, equal maxima keep the
// lower index.  Deterministic for a fixed merge tree.
__device__ __forceinline__ SoftStat softstat_merge(SoftStat x, SoftStat y) {
  SoftStat r;
  r.m = fmaxf(x.m, y.m);
  if (r.m == -INFINITY) return {-INFINITY, 0.0f, min(x.a, y.a)};
  const float sx = (x.m == -INFINITY) ? 0.0f : x.s * expf(x.m - r.m);
  const float sy = (y.m == -INFINITY) ? 0.0f : y.s * expf(y.m - r.m);
  r.s = sx + sy;
  if (x.m > y.m) r.a = x.a;
  else if (y.m > x.m) r.a = y.a;
  else r.a = min(x.a, y.a);
  return r;
}

__device__ __forceinline__ SoftStat shfl_xor_stat(SoftStat v, int o, int width) {
  return {__shfl_xor(v.m, o, width), __shfl_xor(v.s, o, width), __shfl_xor(v.a, o, width)};
}

}  // namespace bdm
