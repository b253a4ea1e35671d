// Grouped expert FFN (SwiGLU) and the weighted combine.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": an expert is gate and up
// at 2,048 by 512 and down at 512 by 2,048 (6.29 MB in BF16); section "The
// expert selection": a block step reads every expert its tokens touch.  At
// 32 tokens a touched routed expert serves ~1.6 tokens, so these kernels are
// weight-streaming: every weight byte is read from HBM exactly once, straight
// into MFMA B-operand registers (16 bytes per lane; one instruction covers a
// 64-byte k-slice of 16 rows), while the few token rows come from L2.
//
// Work is indexed by the list of touched expert groups (the shared expert is
// group E), heaviest first; workgroups past its end exit at once.  A
// workgroup issues its weight loads first and then finds the tokens of its
// expert by scanning the top-k table with wave ballots.  Activations and outputs are stored per
// (token, slot): row t*(k+1)+j for the j-th pick, t*(k+1)+k for the shared
// expert, so the combine reads each token's k+1 rows contiguously.
//
//   gateup_kernel   work item = (expert, 16 columns of I).  8 waves split
//                   K = H; each wave loads its whole K-slice of the 16 gate
//                   and 16 up rows in one burst, multiplies the expert's
//                   token tiles, and the partial sums meet in LDS where
//                   silu(g) * u is formed and stored as bf16.
//   down_kernel     work item = (expert, 64 rows of H).  Each wave owns 16
//                   output rows and the whole K = I; fp32 results per pair.
//   combine_kernel  y_t = bf16(r_t + sum_j w_tj Y_tj + Y_t,shared), fixed
//                   order, no atomics.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

constexpr int kGuCols = 16;     // I columns per gate/up work item
constexpr int kGuWaves = 8;     // waves splitting K in gate/up
constexpr int kGuMaxKs = 8;     // k-steps of 32 per wave: H <= 8 * 8 * 32 = 2048
constexpr int kGuMt = 2;        // 16-token tiles multiplied per pass
constexpr int kDnRows = 64;     // H rows per down work item

// Collect the (token, slot) rows routed to expert e into `rows` (LDS, in
// increasing token order) and return their number.  Called by all threads;
// wave 0 scans, the others wait at the barrier.
__device__ __forceinline__ int gather_pairs(int e, int E, int T, int k,
                                            const int32_t* __restrict__ topk_idx, int* rows) {
  __shared__ int s_count;
  const int K1 = k + 1;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    if (e == E) {
      for (int t = lane; t < T; t += kWave) rows[t] = t * K1 + k;
      if (lane == 0) s_count = T;
    } else {
      const int n = T * k;
      int cnt = 0;
      for (int b = 0; b < n; b += kWave) {
        const int p = b + lane;
        const bool hit = p < n && topk_idx[p] == e;
        const unsigned long long m = __ballot(hit);
        if (hit) {
          const int t = p / k;
          rows[cnt + __popcll(m & ((1ull << lane) - 1ull))] = t * K1 + (p - t * k);
        }
        cnt += __popcll(m);
      }
      if (lane == 0) s_count = cnt;
    }
  }
  __syncthreads();
  return s_count;
}

__global__ __launch_bounds__(kGuWaves * 64, 4) void gateup_kernel(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int k,
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ ws_gate, const uint16_t* __restrict__ ws_up,
    const int32_t* __restrict__ info, const int32_t* __restrict__ touched,
    const int32_t* __restrict__ topk_idx, uint16_t* __restrict__ act) {
  __shared__ f32x4 red[kGuWaves][kGuMt][2][kWave];   // 32 KB
  __shared__ int rows[BDM_MAX_TOKENS];

  const int tiles = I / kGuCols;
  const int gi = blockIdx.x / tiles;
  if (gi >= info[0]) return;                  // past the touched groups
  const int e = touched[gi];
  const int n0 = (blockIdx.x % tiles) * kGuCols;
  const int K1 = k + 1;

  const uint16_t* Wg = (e == E) ? ws_gate : w_gate + static_cast<size_t>(e) * I * H;
  const uint16_t* Wu = (e == E) ? ws_up : w_up + static_cast<size_t>(e) * I * H;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int KS = H / 32;
  const int ksw = (KS + kGuWaves - 1) / kGuWaves;
  const int s0 = wave * ksw;

  // one burst: this wave's K-slice of the 16 gate rows and 16 up rows,
  // issued before the token scan so the scan hides under the loads
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

  const int m = gather_pairs(e, E, T, k, topk_idx, rows);

  for (int mc = 0; mc < m; mc += 16 * kGuMt) {
    f32x4 ag[kGuMt], au[kGuMt];
    const uint16_t* xr[kGuMt];
    bool ok[kGuMt];
#pragma unroll
    for (int mt = 0; mt < kGuMt; ++mt) {
      ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = mc + mt * 16 + c;
      ok[mt] = r < m;
      const int tok = ok[mt] ? rows[r] / K1 : 0;
      xr[mt] = x + static_cast<size_t>(tok) * H + g * 8;
    }
#pragma unroll
    for (int q = 0; q < kGuMaxKs; ++q) {
      const int s = s0 + q;
      if (q < ksw && s < KS) {
#pragma unroll
        for (int mt = 0; mt < kGuMt; ++mt) {
          if (mc + mt * 16 < m) {
            const u32x4 a = ok[mt] ? ld16(xr[mt] + s * 32) : u32x4{0u, 0u, 0u, 0u};
            ag[mt] = mfma_bf16(a, bg[q], ag[mt]);
            au[mt] = mfma_bf16(a, bu[q], au[mt]);
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < kGuMt; ++mt) {
      red[wave][mt][0][lane] = ag[mt];
      red[wave][mt][1][lane] = au[mt];
    }
    __syncthreads();
    if (threadIdx.x < kGuMt * kWave) {
      const int mt = threadIdx.x / kWave;
      const int ln = threadIdx.x % kWave;
      f32x4 gs = red[0][mt][0][ln], us = red[0][mt][1][ln];
#pragma unroll
      for (int w = 1; w < kGuWaves; ++w) {
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
          act[static_cast<size_t>(rows[r]) * I + col] = f32_to_bf16(a);
        }
      }
    }
    __syncthreads();
  }
}

template <int KSMAX>
__global__ __launch_bounds__(256, 2) void down_kernel(
    const uint16_t* __restrict__ act, int T, int H, int I, int E, int k,
    const uint16_t* __restrict__ w_down, const uint16_t* __restrict__ ws_down,
    const int32_t* __restrict__ info, const int32_t* __restrict__ touched,
    const int32_t* __restrict__ topk_idx, float* __restrict__ ypair) {
  __shared__ int rows[BDM_MAX_TOKENS];
  const int tiles = H / kDnRows;
  const int gi = blockIdx.x / tiles;
  if (gi >= info[0]) return;                  // past the touched groups
  const int e = touched[gi];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int n0 = (blockIdx.x % tiles) * kDnRows + wave * 16;
  const int KS = I / 32;

  const uint16_t* Wd = (e == E) ? ws_down : w_down + static_cast<size_t>(e) * H * I;
  u32x4 b[KSMAX];
  const size_t roff = static_cast<size_t>(n0 + c) * I + g * 8;
#pragma unroll
  for (int s = 0; s < KSMAX; ++s)
    b[s] = (s < KS) ? ld16_stream(Wd + roff + s * 32) : u32x4{0u, 0u, 0u, 0u};

  const int m = gather_pairs(e, E, T, k, topk_idx, rows);

  for (int mt = 0; mt * 16 < m; ++mt) {
    const int r = mt * 16 + c;
    const bool ok = r < m;
    const uint16_t* ar = act + static_cast<size_t>(ok ? rows[r] : rows[0]) * I + g * 8;
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
      if (rr < m) ypair[static_cast<size_t>(rows[rr]) * H + n0 + c] = acc[q];
    }
  }
}

// One workgroup per token; a thread owns 8 consecutive columns and issues all
// of its k+1 row loads before summing them in slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypair, int H,
                                                      int k, int has_shared,
                                                      const float* __restrict__ topk_w,
                                                      const uint16_t* residual, uint16_t* y) {
  const int t = blockIdx.x;
  const int h0 = threadIdx.x * 8;
  if (h0 >= H) return;
  const int K1 = k + 1;
  const float* yrow = ypair + static_cast<size_t>(t) * K1 * H + h0;
  float4 v[BDM_MAX_TOPK + 1][2];
#pragma unroll
  for (int j = 0; j <= BDM_MAX_TOPK; ++j) {
    if (j < k || (j == k && has_shared)) {
      v[j][0] = *reinterpret_cast<const float4*>(yrow + static_cast<size_t>(j) * H);
      v[j][1] = *reinterpret_cast<const float4*>(yrow + static_cast<size_t>(j) * H + 4);
    }
  }
  float acc[8];
  if (residual) {
    const u32x4 r = ld16(residual + static_cast<size_t>(t) * H + h0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __uint_as_float(r[i] << 16);
      acc[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j <= BDM_MAX_TOPK; ++j) {
    const float yv[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w,
                         v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
    if (j < k) {
      const float wj = topk_w[t * k + j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, yv[i], acc[i]);
    } else if (j == k && has_shared) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += yv[i];
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(y + static_cast<size_t>(t) * H + h0) = o;
}

void launch_experts(const uint16_t* x, int T, int H, int I, int E, int k, int has_shared,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                    const uint16_t* residual, uint16_t* y, const MoeMeta& meta, hipStream_t s) {
  // upper bound on touched groups; workgroups past the actual count exit at once
  const int groups = (T * k < E ? T * k : E) + (has_shared ? 1 : 0);
  gateup_kernel<<<groups * (I / kGuCols), kGuWaves * 64, 0, s>>>(
      x, T, H, I, E, k, w_gate, w_up, ws_gate, ws_up, meta.info, meta.touched, meta.topk_idx,
      meta.act);
  if (I <= 512) {
    down_kernel<16><<<groups * (H / kDnRows), 256, 0, s>>>(
        meta.act, T, H, I, E, k, w_down, ws_down, meta.info, meta.touched, meta.topk_idx,
        meta.ypair);
  } else {
    down_kernel<32><<<groups * (H / kDnRows), 256, 0, s>>>(
        meta.act, T, H, I, E, k, w_down, ws_down, meta.info, meta.touched, meta.topk_idx,
        meta.ypair);
  }
  combine_kernel<<<T, 256, 0, s>>>(meta.ypair, H, k, has_shared, meta.topk_w, residual, y);
}

}  // namespace bdm
