// RMSNorm between MoE layers: out = bf16(x / sqrt(mean(x^2) + eps) * gamma).
// The pages give no normalisation; this is the pre-norm of the 40-layer
// stack workload (eps 1e-6, unit gamma).  One workgroup per row, fp32 math,
// 8 elements (one 16-byte load) per thread.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, const float* gamma,
                                                      float eps, int H, uint16_t* out) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int i0 = threadIdx.x * 8;
  const bool on = i0 < H;
  float v[8];
  const u32x4 raw = on ? ld16(x + static_cast<size_t>(t) * H + i0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(raw[j] << 16);
    v[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
  }
  const float r = row_rms_scale(v, eps, H, part);
  if (!on) return;
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = v[2 * j] * r, b = v[2 * j + 1] * r;
    if (gamma) {
      a *= gamma[i0 + 2 * j];
      b *= gamma[i0 + 2 * j + 1];
    }
    o[j] = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  }
  *reinterpret_cast<u32x4*>(out + static_cast<size_t>(t) * H + i0) = o;
}

void launch_rmsnorm(const uint16_t* x, const float* gamma, float eps, int T, int H,
                    uint16_t* out, hipStream_t s) {
  rmsnorm_kernel<<<T, 256, 0, s>>>(x, gamma, eps, H, out);
}

}  // namespace bdm
