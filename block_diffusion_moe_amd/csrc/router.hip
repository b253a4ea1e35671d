// Router and top-k selection for the routed MoE layer.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": 256 routed experts, each
// token routed to 8 of them, plus one shared expert that is always on.
//
//   router_kernel  logits l[t][e] = x_t . w_router[e] (+ bias[e]) in fp32.
//                  A small GEMM (T x H) . (H x E) on bf16 MFMA: each fp32
//                  router weight is split exactly into three bf16 terms
//                  (hi + mid + lo == w), so x . w is the fp32-accumulated sum
//                  of exact products, as an fp32 dot product would be.
//                  Workgroup tile: 16 experts x 32 tokens, 16 waves split K
//                  (every load issued before the arithmetic) and meet in LDS.
//   select_kernel  one workgroup: per token (one wave each) softmax over E,
//                  the k largest logits (wave-wide argmax rounds, equal logits
//                  -> lower id) and their renormalised weights; then the list
//                  of touched expert groups (shared first, then experts with
//                  >= 16 tokens, then the rest), which sizes and orders the
//                  expert kernels' work.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

// w == hi + mid + lo exactly, each term a bf16 (the 24-bit fp32 significand
// in three 8-bit pieces; every subtraction below is exact).
__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  lo = f32_to_bf16(r2);
}

constexpr int kRtWaves = 16;    // waves per router workgroup (split K)
constexpr int kRtMaxKs = 4;     // k-steps per wave: H <= 16 * 4 * 32 = 2048

__global__ __launch_bounds__(kRtWaves * 64) void router_kernel(const uint16_t* __restrict__ x,
                                                              int T, int H,
                                                              const float* __restrict__ wr,
                                                              const float* __restrict__ bias,
                                                              int E, float* __restrict__ logits) {
  __shared__ f32x4 red[kRtWaves][2][kWave];   // 32 KB
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const int t0 = blockIdx.y * 32;
  const int KS = H / 32;
  const int ksw = (KS + kRtWaves - 1) / kRtWaves;
  const int s0 = wave * ksw;

  const int er = (e0 + c) < E ? (e0 + c) : (E - 1);
  const float* wrow = wr + static_cast<size_t>(er) * H + g * 8;
  const bool ok0 = (t0 + c) < T;
  const bool ok1 = (t0 + 16 + c) < T;
  const bool two = (t0 + 16) < T;
  const uint16_t* x0 = x + static_cast<size_t>(ok0 ? t0 + c : 0) * H + g * 8;
  const uint16_t* x1 = x + static_cast<size_t>(ok1 ? t0 + 16 + c : 0) * H + g * 8;

  // every load of this wave's K-slice first, then the arithmetic
  float4 wa[kRtMaxKs], wb[kRtMaxKs];
  u32x4 a0[kRtMaxKs], a1[kRtMaxKs];
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    const int s = s0 + q;
    const bool on = q < ksw && s < KS;
    wa[q] = on ? *reinterpret_cast<const float4*>(wrow + s * 32) : float4{0.f, 0.f, 0.f, 0.f};
    wb[q] = on ? *reinterpret_cast<const float4*>(wrow + s * 32 + 4) : float4{0.f, 0.f, 0.f, 0.f};
    a0[q] = (on && ok0) ? ld16(x0 + s * 32) : u32x4{0u, 0u, 0u, 0u};
    a1[q] = (on && ok1) ? ld16(x1 + s * 32) : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    if (q < ksw && s0 + q < KS) {
      const float wv[8] = {wa[q].x, wa[q].y, wa[q].z, wa[q].w, wb[q].x, wb[q].y, wb[q].z, wb[q].w};
      uint16_t hi[8], mi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) split3(wv[j], hi[j], mi[j], lo[j]);
      u32x4 bh, bm, bl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bh[j] = static_cast<uint32_t>(hi[2 * j]) | (static_cast<uint32_t>(hi[2 * j + 1]) << 16);
        bm[j] = static_cast<uint32_t>(mi[2 * j]) | (static_cast<uint32_t>(mi[2 * j + 1]) << 16);
        bl[j] = static_cast<uint32_t>(lo[2 * j]) | (static_cast<uint32_t>(lo[2 * j + 1]) << 16);
      }
      acc0 = mfma_bf16(a0[q], bh, acc0);
      acc0 = mfma_bf16(a0[q], bm, acc0);
      acc0 = mfma_bf16(a0[q], bl, acc0);
      if (two) {
        acc1 = mfma_bf16(a1[q], bh, acc1);
        acc1 = mfma_bf16(a1[q], bm, acc1);
        acc1 = mfma_bf16(a1[q], bl, acc1);
      }
    }
  }
  red[wave][0][lane] = acc0;
  red[wave][1][lane] = acc1;
  __syncthreads();
  if (threadIdx.x < 2 * kWave) {
    const int mt = threadIdx.x / kWave;
    const int ln = threadIdx.x % kWave;
    f32x4 sum = red[0][mt][ln];
#pragma unroll
    for (int w = 1; w < kRtWaves; ++w) sum += red[w][mt][ln];
    const int e = e0 + (ln & 15);
    if (e < E) {
      const float b = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mt * 16 + 4 * (ln >> 4) + i;
        if (t < T) logits[static_cast<size_t>(t) * E + e] = sum[i] + b;
      }
    }
  }
}

// Top-k of one token's logit row, held as PER values per lane (lane + 64*i).
// Returns the j-th pick and weight in lane j (j < k).
template <int PER>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int E, int k, int renorm,
                                         int lane, int& sel_e, float& sel_w) {
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const float l = (e < E) ? row[e] : -INFINITY;
    v[i] = (l == l) ? l : -INFINITY;             // NaN logits rank last
  }
  uint32_t picked = 0u;
  float sel_v = 0.0f, first_v = 0.0f;
  sel_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = INT32_MAX;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !(picked & (1u << i)) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
    wave_argmax(bv, be);
    if ((be % kWave) == lane) picked |= 1u << (be / kWave);
    if (j == 0) first_v = bv;
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  // w_j = exp(l_j - l_max) / (sum over the picks when renormalised, else over all E)
  const float z = (lane < k) ? expf(sel_v - first_v) : 0.0f;
  float den;
  if (renorm) {
    den = wave_sum(z);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      if (e < E) s += expf(v[i] - first_v);
    }
    den = wave_sum(s);
  }
  sel_w = z / den;
}

// One workgroup: top-k of every token (one wave per token at a time), then
// the list of touched expert groups for the expert kernels: the shared
// expert (group E, all T tokens) first, then routed experts with at least 16
// tokens, then the others, each run in increasing id; and its length.
template <int PER>
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ logits, int T,
                                                     int E, int k, int renorm, int has_shared,
                                                     int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w,
                                                     int32_t* __restrict__ info,
                                                     int32_t* __restrict__ touched,
                                                     int32_t* __restrict__ user_idx,
                                                     float* __restrict__ user_w) {
  __shared__ int cnt[BDM_MAX_EXPERTS];
  __shared__ int wtot[2][16];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int nwaves = blockDim.x / kWave;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int t = wave; t < T; t += nwaves) {
    int sel_e;
    float sel_w;
    topk_row<PER>(logits + static_cast<size_t>(t) * E, E, k, renorm, lane, sel_e, sel_w);
    if (lane < k) {
      topk_idx[t * k + lane] = sel_e;
      topk_w[t * k + lane] = sel_w;
      if (user_idx) user_idx[t * k + lane] = sel_e;
      if (user_w) user_w[t * k + lane] = sel_w;
      atomicAdd(&cnt[sel_e], 1);
    }
  }
  __syncthreads();
  // E <= 1024 = blockDim.x: one expert per thread; prefix positions by ballot
  const int e = tid;
  const int ce = (e < E) ? cnt[e] : 0;
  const bool heavy = ce >= 16;
  const bool light = ce > 0 && ce < 16;
  const unsigned long long mh = __ballot(heavy);
  const unsigned long long ml = __ballot(light);
  const unsigned long long below = (1ull << lane) - 1ull;
  if (lane == 0) {
    wtot[0][wave] = __popcll(mh);
    wtot[1][wave] = __popcll(ml);
  }
  __syncthreads();
  int bh = 0, bl = 0, nh = 0, nl = 0;
  for (int w = 0; w < nwaves; ++w) {
    if (w < wave) {
      bh += wtot[0][w];
      bl += wtot[1][w];
    }
    nh += wtot[0][w];
    nl += wtot[1][w];
  }
  const int base = has_shared ? 1 : 0;
  if (heavy) touched[base + bh + __popcll(mh & below)] = e;
  if (light) touched[base + nh + bl + __popcll(ml & below)] = e;
  if (tid == 0) {
    if (has_shared) touched[0] = E;
    info[0] = base + nh + nl;
  }
}

void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, const MoeMeta& meta, int32_t* user_idx,
                   float* user_w, hipStream_t s) {
  const dim3 grid((E + 15) / 16, (T + 31) / 32);
  router_kernel<<<grid, kRtWaves * 64, 0, s>>>(x, T, H, wr, bias, E, meta.logits);
#define BDM_SELECT(P)                                                                          \
  select_kernel<P><<<1, 1024, 0, s>>>(meta.logits, T, E, k, renorm, has_shared, meta.topk_idx, \
                                      meta.topk_w, meta.info, meta.touched, user_idx, user_w)
  if (E <= 256) BDM_SELECT(4);
  else if (E <= 512) BDM_SELECT(8);
  else BDM_SELECT(16);
#undef BDM_SELECT
}

}  // namespace bdm
