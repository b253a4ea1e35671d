// Grouped expert FFN (SwiGLU) and the weighted combine.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": an expert is gate and up
// at 2,048 by 512 and down at 512 by 2,048 (6.29 MB in BF16); section "The
// expert selection": a block step reads every expert its tokens touch.  At
// 32 tokens a touched routed expert serves ~1.6 tokens, so these kernels are
// weight-streaming: every weight byte is read from HBM exactly once, straight
// into MFMA B-operand registers (16 bytes per lane, the 16 rows of a 64-byte
// k-slice per instruction), while the few token rows come from L2.
//
//   gateup_kernel   work item = (touched group, 16 columns of I).  The 4
//                   waves split K = H; each wave holds its whole K-slice of
//                   the 16 gate rows and 16 up rows in registers (one
//                   burst of loads), multiplies every 16-token tile of the
//                   group's tokens, and the partial sums meet in LDS where
//                   silu(g) * u is formed and stored as bf16.
//   down_kernel     work item = (touched group, 64 rows of H).  Each wave
//                   owns 16 output rows and the whole K = I; results are
//                   fp32 per (token, expert) pair.
//   combine_kernel  y_t = bf16(r_t + sum_j w_tj Y_tj + Y_t,shared), fixed
//                   order, no atomics.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

constexpr int kGuCols = 16;     // I columns per gate/up work item
constexpr int kGuMaxKs = 16;    // k-steps of 32 per wave: H <= 4 * 16 * 32 = 2048
constexpr int kDnRows = 64;     // H rows per down work item

__global__ __launch_bounds__(256, 2) void gateup_kernel(
    const uint16_t* __restrict__ x, int H, int I, int E, const uint16_t* __restrict__ w_gate,
    const uint16_t* __restrict__ w_up, const uint16_t* __restrict__ ws_gate,
    const uint16_t* __restrict__ ws_up, const int32_t* __restrict__ info,
    const int32_t* __restrict__ touched, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ pair_token, uint16_t* __restrict__ act) {
  __shared__ f32x4 red[4][4][2][kWave];   // [wave][m-tile][gate/up][lane]  32 KB

  const int tiles = I / kGuCols;
  const int item = blockIdx.x;
  if (item >= info[0] * tiles) return;
  const int e = touched[item / tiles];
  const int n0 = (item % tiles) * kGuCols;
  const int p0 = offs[e];
  const int m = offs[e + 1] - p0;

  const uint16_t* Wg = (e == E) ? ws_gate : w_gate + static_cast<size_t>(e) * I * H;
  const uint16_t* Wu = (e == E) ? ws_up : w_up + static_cast<size_t>(e) * I * H;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int KS = H / 32;
  const int ksw = (KS + 3) / 4;
  const int s0 = wave * ksw;

  // One burst: this wave's K-slice of 16 gate rows and 16 up rows.
  u32x4 bg[kGuMaxKs], bu[kGuMaxKs];
  const size_t roff = static_cast<size_t>(n0 + c) * H + g * 8;
#pragma unroll
  for (int q = 0; q < kGuMaxKs; ++q) {
    const int s = s0 + q;
    if (q < ksw && s < KS) {
      bg[q] = ld16_stream(Wg + roff + s * 32);
      bu[q] = ld16_stream(Wu + roff + s * 32);
    } else {
      bg[q] = u32x4{0u, 0u, 0u, 0u};
      bu[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  for (int mc = 0; mc < m; mc += 64) {
    f32x4 ag[4], au[4];
    const uint16_t* xr[4];
    bool ok[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = mc + mt * 16 + c;
      ok[mt] = r < m;
      const int tok = ok[mt] ? pair_token[p0 + r] : 0;
      xr[mt] = x + static_cast<size_t>(tok) * H + g * 8;
    }
#pragma unroll
    for (int q = 0; q < kGuMaxKs; ++q) {
      const int s = s0 + q;
      if (q < ksw && s < KS) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mc + mt * 16 < m) {
            const u32x4 a = ok[mt] ? ld16(xr[mt] + s * 32) : u32x4{0u, 0u, 0u, 0u};
            ag[mt] = mfma_bf16(a, bg[q], ag[mt]);
            au[mt] = mfma_bf16(a, bu[q], au[mt]);
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      red[wave][mt][0][lane] = ag[mt];
      red[wave][mt][1][lane] = au[mt];
    }
    __syncthreads();
    {
      const int mt = threadIdx.x / kWave;   // 4 m-tiles x 64 lanes = 256 threads
      const int ln = threadIdx.x % kWave;
      f32x4 gs = red[0][mt][0][ln], us = red[0][mt][1][ln];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        gs += red[w][mt][0][ln];
        us += red[w][mt][1][ln];
      }
      const int col = n0 + (ln & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = mc + mt * 16 + 4 * (ln >> 4) + q;
        if (r < m) {
          const float gv = gs[q];
          const float a = gv / (1.0f + expf(-gv)) * us[q];
          act[static_cast<size_t>(p0 + r) * I + col] = f32_to_bf16(a);
        }
      }
    }
    __syncthreads();
  }
}

template <int KSMAX>
__global__ __launch_bounds__(256, 2) void down_kernel(
    const uint16_t* __restrict__ act, int H, int I, int E, const uint16_t* __restrict__ w_down,
    const uint16_t* __restrict__ ws_down, const int32_t* __restrict__ info,
    const int32_t* __restrict__ touched, const int32_t* __restrict__ offs,
    float* __restrict__ ypair) {
  const int tiles = H / kDnRows;
  const int item = blockIdx.x;
  if (item >= info[0] * tiles) return;
  const int e = touched[item / tiles];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int n0 = (item % tiles) * kDnRows + wave * 16;
  const int p0 = offs[e];
  const int m = offs[e + 1] - p0;
  const int KS = I / 32;

  const uint16_t* Wd = (e == E) ? ws_down : w_down + static_cast<size_t>(e) * H * I;
  u32x4 b[KSMAX];
  const size_t roff = static_cast<size_t>(n0 + c) * I + g * 8;
#pragma unroll
  for (int s = 0; s < KSMAX; ++s)
    b[s] = (s < KS) ? ld16_stream(Wd + roff + s * 32) : u32x4{0u, 0u, 0u, 0u};

  for (int mt = 0; mt * 16 < m; ++mt) {
    const int r = mt * 16 + c;
    const bool ok = r < m;
    const uint16_t* ar = act + static_cast<size_t>(p0 + (ok ? r : 0)) * I + g * 8;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSMAX; ++s) {
      if (s < KS) {
        const u32x4 a = ok ? ld16(ar + s * 32) : u32x4{0u, 0u, 0u, 0u};
        acc = mfma_bf16(a, b[s], acc);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = mt * 16 + 4 * g + q;
      if (rr < m) ypair[static_cast<size_t>(p0 + rr) * H + n0 + c] = acc[q];
    }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypair, int H,
                                                      int k, int has_shared,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ topk_w,
                                                      const uint16_t* residual, uint16_t* y) {
  const int t = blockIdx.x;
  const int K1 = k + 1;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float acc = residual ? bf16_to_f32(residual[static_cast<size_t>(t) * H + h]) : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int p = pos[t * K1 + j];
      acc = fmaf(topk_w[t * k + j], ypair[static_cast<size_t>(p) * H + h], acc);
    }
    if (has_shared) acc += ypair[static_cast<size_t>(pos[t * K1 + k]) * H + h];
    y[static_cast<size_t>(t) * H + h] = f32_to_bf16(acc);
  }
}

void launch_experts(const uint16_t* x, int T, int H, int I, int E, int k, int has_shared,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                    const uint16_t* residual, uint16_t* y, const MoeMeta& meta, hipStream_t s) {
  const int max_groups = (T * k < E ? T * k : E) + (has_shared ? 1 : 0);
  gateup_kernel<<<max_groups * (I / kGuCols), 256, 0, s>>>(
      x, H, I, E, w_gate, w_up, ws_gate, ws_up, meta.info, meta.touched, meta.offs,
      meta.pair_token, meta.act);
  if (I <= 512) {
    down_kernel<16><<<max_groups * (H / kDnRows), 256, 0, s>>>(
        meta.act, H, I, E, w_down, ws_down, meta.info, meta.touched, meta.offs, meta.ypair);
  } else {
    down_kernel<32><<<max_groups * (H / kDnRows), 256, 0, s>>>(
        meta.act, H, I, E, w_down, ws_down, meta.info, meta.touched, meta.offs, meta.ypair);
  }
  combine_kernel<<<T, 256, 0, s>>>(meta.ypair, H, k, has_shared, meta.pos, meta.topk_w, residual,
                                   y);
}

}  // namespace bdm
