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
//                  Workgroup tile: 16 experts x 32 tokens x one of 4 K-parts
//                  (4 waves split the part, every load issued first); the
//                  parts are summed in order by the select step.
//   select_kernel  per token (one wave each): softmax over E, the k largest
//                  logits (wave-wide argmax rounds, equal logits -> lower id)
//                  and their renormalised weights; the last workgroup to
//                  finish groups the picks by expert (slot table + pair rows)
//                  for the expert kernels.
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

constexpr int kRtWaves = 4;     // waves per router workgroup
constexpr int kRtMaxKs = 4;     // k-steps per wave: H <= kRouterParts * 4 * 4 * 32 = 2048

// Partial logits over one K-part: part[z][t][e] = sum_{h in part z} x[t][h] w[e][h].
// The fp32 partials are summed (in part order) with the bias by the select
// step.  Block (0,0,0) also clears the select step's completion ticket.
__global__ __launch_bounds__(kRtWaves * 64) void router_kernel(const uint16_t* __restrict__ x,
                                                              int T, int H,
                                                              const float* __restrict__ wr, int E,
                                                              float* __restrict__ part,
                                                              int32_t* __restrict__ ticket) {
  __shared__ f32x4 red[kRtWaves][2][kWave];
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *ticket = 0;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const int t0 = blockIdx.y * 32;
  const int z = blockIdx.z;
  const int KS = H / 32;
  const int ksp = (KS + kRouterParts - 1) / kRouterParts;       // k-steps of this part
  const int ksw = (ksp + kRtWaves - 1) / kRtWaves;
  const int s0 = z * ksp + wave * ksw;
  const int s1 = min(min(s0 + ksw, (z + 1) * ksp), KS);

  const int er = (e0 + c) < E ? (e0 + c) : (E - 1);
  const float* wrow = wr + static_cast<size_t>(er) * H + g * 8;
  const bool ok0 = (t0 + c) < T;
  const bool ok1 = (t0 + 16 + c) < T;
  const bool two = (t0 + 16) < T;
  const uint16_t* x0 = x + static_cast<size_t>(ok0 ? t0 + c : 0) * H + g * 8;
  const uint16_t* x1 = x + static_cast<size_t>(ok1 ? t0 + 16 + c : 0) * H + g * 8;

  // every load of this wave's K-slice first (clamped, no branches), then math
  float4 wa[kRtMaxKs], wb[kRtMaxKs];
  u32x4 a0[kRtMaxKs], a1[kRtMaxKs];
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    const int s = (s0 + q < s1) ? s0 + q : 0;
    wa[q] = *reinterpret_cast<const float4*>(wrow + s * 32);
    wb[q] = *reinterpret_cast<const float4*>(wrow + s * 32 + 4);
    a0[q] = ld16(x0 + s * 32);
    a1[q] = ld16(x1 + s * 32);
  }
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    if (s0 + q < s1) {
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
      const u32x4 z0 = ok0 ? a0[q] : u32x4{0u, 0u, 0u, 0u};
      acc0 = mfma_bf16(z0, bh, acc0);
      acc0 = mfma_bf16(z0, bm, acc0);
      acc0 = mfma_bf16(z0, bl, acc0);
      if (two) {
        const u32x4 z1 = ok1 ? a1[q] : u32x4{0u, 0u, 0u, 0u};
        acc1 = mfma_bf16(z1, bh, acc1);
        acc1 = mfma_bf16(z1, bm, acc1);
        acc1 = mfma_bf16(z1, bl, acc1);
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
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mt * 16 + 4 * (ln >> 4) + i;
        if (t < T) part[(static_cast<size_t>(z) * T + t) * E + e] = sum[i];
      }
    }
  }
}

// Top-k of one token's logit row, held as PER values per lane (lane + 64*i).
// Returns the j-th pick and weight in lane j (j < k).
template <int PER>
__device__ __forceinline__ void topk_row(const float* __restrict__ part, size_t zstride,
                                         const float* __restrict__ bias, int E, int k,
                                         int renorm, int lane, int& sel_e, float& sel_w) {
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const int ec = e < E ? e : 0;
    float l = part[ec];
#pragma unroll
    for (int z = 1; z < kRouterParts; ++z) l += part[z * zstride + ec];
    if (bias) l += bias[ec];
    l = (e < E) ? l : -INFINITY;
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

constexpr int kSelWaves = 4;    // tokens per select workgroup (one wave each)

// Top-k of every token (one wave per token, kSelWaves tokens per workgroup).
// The last workgroup to finish (completion ticket) then groups the picks by
// expert for the expert kernels:
//   slots[i] = {expert, offset, count, 0} for the i-th touched group -- the
//              shared expert (group E, all T tokens) first, then routed
//              experts with at least 16 tokens, then the others, each run in
//              increasing id -- and {-1, 0, 0, 0} for i = n .. E;
//   pair_rows[offset .. offset+count) = the (token, slot) rows t*(k+1)+j of
//              the group's tokens (shared: t*(k+1)+k).
// The order inside a group is whatever the LDS atomics produce; every row's
// result is computed independently of the others, so outputs do not depend
// on it.
template <int PER>
__global__ __launch_bounds__(kSelWaves * 64) void select_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int T, int E, int k,
    int renorm, int has_shared, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* ticket, int4* __restrict__ slots, int32_t* __restrict__ pair_rows,
    int32_t* __restrict__ info, int32_t* __restrict__ user_idx, float* __restrict__ user_w) {
  __shared__ int cnt[BDM_MAX_EXPERTS + 1];
  __shared__ int eoff[BDM_MAX_EXPERTS + 1];
  __shared__ int wtot[2][kSelWaves];
  __shared__ int s_last, s_carry[3];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int K1 = k + 1;

  const int t = blockIdx.x * kSelWaves + wave;
  if (t < T) {
    int sel_e;
    float sel_w;
    topk_row<PER>(part + static_cast<size_t>(t) * E, static_cast<size_t>(T) * E, bias, E, k,
                  renorm, lane, sel_e, sel_w);
    if (lane < k) {
      topk_idx[t * k + lane] = sel_e;
      topk_w[t * k + lane] = sel_w;
      if (user_idx) user_idx[t * k + lane] = sel_e;
      if (user_w) user_w[t * k + lane] = sel_w;
    }
  }
  // publish this workgroup's picks, then take a ticket
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(ticket, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- the last workgroup: group the T*k picks by expert ----------------
  for (int e = tid; e <= E; e += blockDim.x) cnt[e] = (e == E) ? (has_shared ? T : 0) : 0;
  __syncthreads();
  for (int p = tid; p < T * k; p += blockDim.x) atomicAdd(&cnt[topk_idx[p]], 1);
  if (tid == 0) {
    s_carry[0] = 0;
    s_carry[1] = 0;
  }
  __syncthreads();
  // two passes over the routed experts in id order (chunks of blockDim.x):
  // first the heavy ones (>= 16 tokens), then the light ones; each touched
  // expert gets its slot position and its pair offset
  const int base = has_shared ? 1 : 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int c0 = 0; c0 < E; c0 += blockDim.x) {
      const int e = c0 + tid;
      const int ce = (e < E) ? cnt[e] : 0;
      const bool in = pass == 0 ? ce >= 16 : (ce > 0 && ce < 16);
      const unsigned long long mk = __ballot(in);
      // pair-count prefix inside the wave (DPP-free: a short serial scan of
      // the wave's counts through LDS is not needed, use ballot-weighted sums)
      int csum = in ? ce : 0;
      int incl = csum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      if (lane == kWave - 1) {
        wtot[0][wave] = __popcll(mk);
        wtot[1][wave] = incl;
      }
      __syncthreads();
      int pos_b = 0, off_b = 0, pos_n = 0, off_n = 0;
      for (int w = 0; w < kSelWaves; ++w) {
        if (w < wave) {
          pos_b += wtot[0][w];
          off_b += wtot[1][w];
        }
        pos_n += wtot[0][w];
        off_n += wtot[1][w];
      }
      if (in) {
        const int pos = base + s_carry[0] + pos_b + __popcll(mk & ((1ull << lane) - 1ull));
        const int off = (has_shared ? T : 0) + s_carry[1] + off_b + incl - csum;
        slots[pos] = int4{e, off, ce, 0};
        eoff[e] = off;
      }
      __syncthreads();
      if (tid == 0) {
        s_carry[0] += pos_n;
        s_carry[1] += off_n;
      }
      __syncthreads();
    }
  }
  const int n = base + s_carry[0];
  if (has_shared && tid == 0) slots[0] = int4{E, 0, T, 0};
  for (int i = n + tid; i <= E; i += blockDim.x) slots[i] = int4{-1, 0, 0, 0};
  if (tid == 0) info[0] = n;
  // scatter the pairs
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < T * k; p += blockDim.x) {
    const int e = topk_idx[p];
    const int tt = p / k;
    pair_rows[eoff[e] + atomicAdd(&cnt[e], 1)] = tt * K1 + (p - tt * k);
  }
  if (has_shared)
    for (int tt = tid; tt < T; tt += blockDim.x) pair_rows[tt] = tt * K1 + k;
}

void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, const MoeMeta& meta, int32_t* user_idx,
                   float* user_w, hipStream_t s) {
  const dim3 grid((E + 15) / 16, (T + 31) / 32, kRouterParts);
  router_kernel<<<grid, kRtWaves * 64, 0, s>>>(x, T, H, wr, E, meta.logits, meta.ticket);
  const int nsel = (T + kSelWaves - 1) / kSelWaves;
#define BDM_SELECT(P)                                                                           \
  select_kernel<P><<<nsel, kSelWaves * 64, 0, s>>>(meta.logits, bias, T, E, k, renorm,         \
                                                   has_shared, meta.topk_idx, meta.topk_w,     \
                                                   meta.ticket, meta.slots, meta.pair_rows,    \
                                                   meta.info, user_idx, user_w)
  if (E <= 256) BDM_SELECT(4);
  else if (E <= 512) BDM_SELECT(8);
  else BDM_SELECT(16);
#undef BDM_SELECT
}

}  // namespace bdm
