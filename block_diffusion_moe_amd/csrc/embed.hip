// Embedding rows of the block's current tokens, the input of every denoise
// step (page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a
// second, read from its files", section "How it writes": each step runs the
// model over the whole block as it stands).
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

// one workgroup per token, thread i holding the row's elements 8i .. 8i+7 (H
// <= 2048 = 256 x 8): the row is copied and normalised as the RMSNorm kernel
// normalises it (the same thread map and summation order, eps 1e-6)
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ w, int V, int H,
                                                    uint16_t* __restrict__ x,
                                                    uint16_t* __restrict__ xn) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  // an id outside the vocabulary reads the nearest row (and is reported in
  // the debug build)
  const int tid_raw = tokens[t];
  if ((tid_raw < 0 || tid_raw >= V) && threadIdx.x == 0) note_oob(kChkTokenId);
  const int id = tid_raw < 0 ? 0 : (tid_raw >= V ? V - 1 : tid_raw);
  const int i0 = threadIdx.x * 8;
  const bool on = i0 < H;
  const u32x4 raw = on ? ld16(w + static_cast<size_t>(id) * H + i0) : u32x4{0u, 0u, 0u, 0u};
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(raw[j] << 16);
    v[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
  }
  const float r = row_rms_scale(v, 1e-6f, H, part);
  if (!on) return;
  *reinterpret_cast<u32x4*>(x + static_cast<size_t>(t) * H + i0) = raw;
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = static_cast<uint32_t>(f32_to_bf16(v[2 * j] * r)) |
           (static_cast<uint32_t>(f32_to_bf16(v[2 * j + 1] * r)) << 16);
  *reinterpret_cast<u32x4*>(xn + static_cast<size_t>(t) * H + i0) = o;
}

void launch_embed(const int32_t* tokens, int T, const uint16_t* w_embed, int V, int H,
                  uint16_t* x, uint16_t* xn, hipStream_t s) {
  embed_kernel<<<T, 256, 0, s>>>(tokens, w_embed, V, H, x, xn);
}

BDM_DEBUG_WORD_READER(debug_words_embed)

}  // namespace bdm
