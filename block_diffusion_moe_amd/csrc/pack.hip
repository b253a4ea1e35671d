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
// The gate/up pair layout interleaves the 16-row groups of two matrices, so
// that the gate and up rows a gate/up work item multiplies lie side by side.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

// one wave per tile; 4 tiles per workgroup.  Group rg goes to group slot
// gm * rg + go of dst (gm = 1, go = 0: the plain layout; gm = 2: gate and up
// groups alternating, see launch_pack_pair).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src, long R, int K,
                                                   uint16_t* __restrict__ dst, long ntiles, int gm,
                                                   int go) {
  const long tile = static_cast<long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x % kWave;
  const int KS = K / 32;
  const long rg = tile / KS;
  const int s = static_cast<int>(tile - rg * KS);
  const long r = rg * 16 + (lane & 15);
  const u32x4 v = (r < R) ? ld16(src + r * K + s * 32 + (lane >> 4) * 8) : u32x4{0u, 0u, 0u, 0u};
  const long out_tile = (rg * gm + go) * KS + s;
  *reinterpret_cast<u32x4*>(dst + (out_tile * kWave + lane) * 8) = v;
}

void launch_pack(const uint16_t* src, long R, int K, uint16_t* dst, hipStream_t s) {
  const long ntiles = ((R + 15) / 16) * (K / 32);
  const long blocks = (ntiles + 3) / 4;
  pack_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(src, R, K, dst, ntiles, 1, 0);
}

// gate and up [R][K] (R % 16 == 0) into one buffer whose 16-row groups
// alternate: group 2g = gate group g, group 2g + 1 = up group g
void launch_pack_pair(const uint16_t* gate, const uint16_t* up, long R, int K, uint16_t* dst,
                      hipStream_t s) {
  const long ntiles = (R / 16) * (K / 32);
  const long blocks = (ntiles + 3) / 4;
  pack_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(gate, R, K, dst, ntiles, 2, 0);
  pack_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(up, R, K, dst, ntiles, 2, 1);
}

}  // namespace bdm
