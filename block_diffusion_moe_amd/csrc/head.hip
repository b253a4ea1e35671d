// Untied output head fused with the low-confidence unmask rule.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": the untied head holds
// 508,559,360 parameters and is read in full at every step; section "How it
// writes", steps 2-3: per slot the most likely token and its probability
// with the mask token's logit at minus infinity, then commit every
// still-masked slot at or above the threshold, else the most confident one.
//
//   head_tile_kernel   one workgroup per 256 vocabulary rows (4 waves x 64).
//                      The weight rows stream from HBM once into MFMA B
//                      registers; the block's hidden states (<= 32 rows per
//                      pass, L2-resident) are the A operand.  The logits never
//                      leave registers: each (token, tile) keeps only the
//                      online-softmax triple (max, sum of exp, argmax).
//   head_merge_kernel  one workgroup: merges the triples of all tiles in a
//                      fixed tree per token -> conf = 1 / sum, argmax; then
//                      applies the commit rule and its progress fallback.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

constexpr int kHeadGroups = 4;   // 16-row vocabulary groups per wave
constexpr int kHeadUnroll = 4;   // k-steps of loads issued together

__global__ __launch_bounds__(256, 2) void head_tile_kernel(
    const uint16_t* __restrict__ h, int H, const uint16_t* __restrict__ w, int V,
    int32_t mask_id, int tok0, int ntok, int ntiles, float* __restrict__ pm,
    float* __restrict__ ps, int32_t* __restrict__ pa) {
  __shared__ SoftStat wres[4][kHeadTokChunk];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int vbase = tile * kHeadTileRows + wave * (kHeadGroups * 16);

  const uint16_t* wrow[kHeadGroups];
#pragma unroll
  for (int q = 0; q < kHeadGroups; ++q) {
    int v = vbase + q * 16 + c;
    v = v < V ? v : V - 1;                      // ragged tail: load a valid row, drop later
    wrow[q] = w + static_cast<size_t>(v) * H + g * 8;
  }
  const uint16_t* hrow[2];
  bool ok[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = mt * 16 + c;
    ok[mt] = r < ntok;
    hrow[mt] = h + static_cast<size_t>(tok0 + (ok[mt] ? r : 0)) * H + g * 8;
  }
  const bool two = ntok > 16;

  f32x4 acc[kHeadGroups][2];
#pragma unroll
  for (int q = 0; q < kHeadGroups; ++q)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KS = H / 32;
  for (int s0 = 0; s0 < KS; s0 += kHeadUnroll) {
    u32x4 b[kHeadUnroll][kHeadGroups];
    u32x4 a[kHeadUnroll][2];
#pragma unroll
    for (int u = 0; u < kHeadUnroll; ++u) {
      const int s = s0 + u;
#pragma unroll
      for (int q = 0; q < kHeadGroups; ++q)
        b[u][q] = (s < KS) ? ld16_stream(wrow[q] + s * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        a[u][mt] = (s < KS && ok[mt]) ? ld16(hrow[mt] + s * 32) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kHeadUnroll; ++u) {
#pragma unroll
      for (int q = 0; q < kHeadGroups; ++q) {
        acc[q][0] = mfma_bf16(a[u][0], b[u][q], acc[q][0]);
        if (two) acc[q][1] = mfma_bf16(a[u][1], b[u][q], acc[q][1]);
      }
    }
  }

  // Epilogue: lane holds vocabulary column c of each group, tokens 4g+i of
  // each m-tile.  Reduce over its 4 groups, then over the 16 lanes of g.
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      SoftStat st = softstat_empty();
#pragma unroll
      for (int q = 0; q < kHeadGroups; ++q) {
        const int v = vbase + q * 16 + c;
        if (v < V && v != mask_id) {
          const float l = acc[q][mt][i];
          if (l > st.m) {
            st.s = (st.m == -INFINITY ? 0.0f : st.s * expf(st.m - l)) + 1.0f;
            st.m = l;
            st.a = v;
          } else {
            st.s += expf(l - st.m);
          }
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) st = softstat_merge(st, shfl_xor_stat(st, o, kWave));
      if (c == 0) wres[wave][mt * 16 + 4 * g + i] = st;
    }
  }
  __syncthreads();
  if (threadIdx.x < ntok) {
    const int r = threadIdx.x;
    SoftStat st = wres[0][r];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) st = softstat_merge(st, wres[wv][r]);
    const size_t o = static_cast<size_t>(tok0 + r) * ntiles + tile;
    pm[o] = st.m;
    ps[o] = st.s;
    pa[o] = st.a;
  }
}

__global__ __launch_bounds__(1024) void head_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const int32_t* __restrict__ pa,
    int T, int ntiles, int32_t mask_id, float threshold, int fallback, int32_t* tokens,
    int32_t* __restrict__ argmax_out, float* __restrict__ conf_out,
    int32_t* __restrict__ n_committed) {
  extern __shared__ float smem[];
  float* sconf = smem;                                   // [T]
  int* sarg = reinterpret_cast<int*>(smem + T);         // [T]
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int nwaves = blockDim.x / kWave;

  for (int t = wave; t < T; t += nwaves) {
    SoftStat st = softstat_empty();
    const size_t base = static_cast<size_t>(t) * ntiles;
    for (int i = lane; i < ntiles; i += kWave)
      st = softstat_merge(st, SoftStat{pm[base + i], ps[base + i], pa[base + i]});
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) st = softstat_merge(st, shfl_xor_stat(st, o, kWave));
    if (lane == 0) {
      const float cf = 1.0f / st.s;
      sconf[t] = cf;
      sarg[t] = st.a;
      if (argmax_out) argmax_out[t] = st.a;
      if (conf_out) conf_out[t] = cf;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // Commit rule, one wave.  Best masked row for the fallback: largest conf,
  // equal -> lowest position.
  int ncommit = 0;
  float best_c = -INFINITY;
  int best_t = INT32_MAX;
  for (int t0 = 0; t0 < T; t0 += kWave) {
    const int t = t0 + lane;
    int commit = 0;
    if (t < T && tokens[t] == mask_id) {
      const float cf = sconf[t];
      if (cf >= threshold) commit = 1;
      if (cf > best_c || (cf == best_c && t < best_t)) {
        best_c = cf;
        best_t = t;
      }
    }
    if (commit) tokens[t] = sarg[t];
    int cnt = commit;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
    ncommit += cnt;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float oc = __shfl_xor(best_c, o, kWave);
    const int ot = __shfl_xor(best_t, o, kWave);
    if (oc > best_c || (oc == best_c && ot < best_t)) {
      best_c = oc;
      best_t = ot;
    }
  }
  if (fallback && ncommit == 0 && best_t != INT32_MAX) {
    if (lane == 0) tokens[best_t] = sarg[best_t];
    ncommit = 1;
  }
  if (lane == 0 && n_committed) *n_committed = ncommit;
}

void launch_head(const uint16_t* h, int T, int H, const uint16_t* w, int V, int32_t mask_id,
                 float threshold, int fallback, int32_t* tokens, int32_t* argmax, float* conf,
                 int32_t* n_committed, const HeadParts& parts, hipStream_t s) {
  const int ntiles = (V + kHeadTileRows - 1) / kHeadTileRows;
  for (int t0 = 0; t0 < T; t0 += kHeadTokChunk) {
    const int n = (T - t0) < kHeadTokChunk ? (T - t0) : kHeadTokChunk;
    head_tile_kernel<<<ntiles, 256, 0, s>>>(h, H, w, V, mask_id, t0, n, ntiles, parts.m, parts.s,
                                            parts.a);
  }
  head_merge_kernel<<<1, 1024, static_cast<size_t>(T) * 8, s>>>(
      parts.m, parts.s, parts.a, T, ntiles, mask_id, threshold, fallback, tokens, argmax, conf,
      n_committed);
}

}  // namespace bdm
