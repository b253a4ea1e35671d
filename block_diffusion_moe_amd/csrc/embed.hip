// Embedding rows of the block's current tokens, the input of every denoise
// step (page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a
// second, read from its files", section "How it writes": each step runs the
// model over the whole block as it stands).
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

// one workgroup per token; 16 bytes per thread per round
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ w, int V, int H,
                                                    uint16_t* __restrict__ x) {
  const int t = blockIdx.x;
  int id = tokens[t];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const uint16_t* src = w + static_cast<size_t>(id) * H;
  uint16_t* dst = x + static_cast<size_t>(t) * H;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8)
    *reinterpret_cast<u32x4*>(dst + c) = ld16(src + c);
}

void launch_embed(const int32_t* tokens, int T, const uint16_t* w_embed, int V, int H,
                  uint16_t* x, hipStream_t s) {
  embed_kernel<<<T, 256, 0, s>>>(tokens, w_embed, V, H, x);
}

}  // namespace bdm
