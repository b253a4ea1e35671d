// Packing of bf16 weight matrices into the MFMA-tile layout.
//
// A row-major matrix W[R][K] (K % 32 == 0) becomes ceil(R/16) x K/32 tiles of
// 1 KB; tile (rg, s) holds rows 16*rg .. 16*rg+15 and k = 32*s .. 32*s+31 in
// the register order of a v_mfma_f32_16x16x32_bf16 operand:
//
//   packed[((rg * (K/32) + s) * 64 + lane) * 8 + i] = W[16*rg + (lane % 16)][32*s + 8*(lane / 16) + i]
//
// (rows past R are zero).  A wave then reads one operand fragment with one
// 1 KB contiguous load, and a 16-row group over all of K is one contiguous
// 32*K-byte run, which the weight-streaming kernels read front to back.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

// one wave per tile; 4 tiles per workgroup
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src, long R, int K,
                                                   uint16_t* __restrict__ dst, long ntiles) {
  const long tile = static_cast<long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x % kWave;
  const int KS = K / 32;
  const long rg = tile / KS;
  const int s = static_cast<int>(tile - rg * KS);
  const long r = rg * 16 + (lane & 15);
  const u32x4 v = (r < R) ? ld16(src + r * K + s * 32 + (lane >> 4) * 8) : u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(dst + (tile * kWave + lane) * 8) = v;
}

void launch_pack(const uint16_t* src, long R, int K, uint16_t* dst, hipStream_t s) {
  const long ntiles = ((R + 15) / 16) * (K / 32);
  const long blocks = (ntiles + 3) / 4;
  pack_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(src, R, K, dst, ntiles);
}

}  // namespace bdm
