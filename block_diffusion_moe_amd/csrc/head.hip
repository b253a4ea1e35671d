// Untied output head fused with the low-confidence unmask rule.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": the untied head holds
// 508,559,360 parameters and is read in full at every step; section "How it
// writes", steps 2-3: per slot the most likely token and its probability
// with the mask token's logit at minus infinity, then commit every
// still-masked slot at or above the threshold, else the most confident one.
//
//   head_tile_kernel   persistent, one workgroup per CU.  The weight rows
//                      stream from HBM once into MFMA B registers; the block's
//                      hidden states (<= 32 rows per pass) sit in LDS as the
//                      A operand.  The logits never leave registers: each
//                      (token, workgroup) keeps only the online-softmax triple
//                      (max, sum of exp, argmax).
//   head_merge_kernel  one workgroup: merges the triples of all workgroups in
//                      a fixed tree per token -> conf = 1 / sum, argmax; then
//                      applies the commit rule and its progress fallback.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

#ifndef BDM_HEAD_UNROLL
#define BDM_HEAD_UNROLL 4
#endif
#ifndef BDM_HEAD_NT
#define BDM_HEAD_NT 1
#endif
#ifndef BDM_HEAD_PREFETCH
#define BDM_HEAD_PREFETCH 1
#endif

constexpr int kHeadGroups = 4;                 // 16-row vocabulary groups a wave multiplies together
constexpr int kHeadUnroll = BDM_HEAD_UNROLL;   // k-steps of weight loads issued together
constexpr int kHeadPad = 8;                    // bf16 padding per staged row (bank spread)

size_t head_lds_bytes(int H) {
  return static_cast<size_t>(kHeadTokChunk) * (H + kHeadPad) * sizeof(uint16_t) +
         static_cast<size_t>(kHeadWaves) * kHeadTokChunk * sizeof(SoftStat);
}

__device__ __forceinline__ u32x4 head_ld(const uint16_t* p) {
  return BDM_HEAD_NT ? ld16_stream(p) : ld16(p);
}

// Loads of one batch: kHeadUnroll k-steps of the four 16-row groups of the
// chunk starting at group gb (groups past the run end, or k past H, load 0).
__device__ __forceinline__ void head_load_batch(u32x4 (&b)[kHeadUnroll][kHeadGroups],
                                                const uint16_t* __restrict__ w, int V, int H,
                                                int gb, int nq, int s0, int KS, int c, int g) {
#pragma unroll
  for (int q = 0; q < kHeadGroups; ++q) {
    int v = (gb + q) * 16 + c;
    v = v < V ? v : V - 1;                      // ragged tail: a valid row, dropped later
    const uint16_t* row = w + static_cast<size_t>(v) * H + g * 8;
#pragma unroll
    for (int u = 0; u < kHeadUnroll; ++u)
      b[u][q] = (q < nq && s0 + u < KS) ? head_ld(row + (s0 + u) * 32) : u32x4{0u, 0u, 0u, 0u};
  }
}

// Persistent: one workgroup per CU, 8 waves.  The <= 32 hidden rows of this
// pass are staged once in LDS (A operand).  The vocabulary is cut into
// 16-row groups and every wave of the grid takes one contiguous run of
// groups (lengths differ by at most one group), streaming those weight rows
// once from HBM as the B operand, four groups (a chunk) at a time.  The loop
// runs over (chunk, k-batch) pairs with the next batch's loads issued before
// the current batch's MFMAs, so a wave always has a batch in flight, also
// across chunk boundaries.  Each lane keeps online-softmax state for its 8
// (token, column) slots across the run; the per-wave results are merged
// across lanes and waves in a fixed order and written as one partial per
// (token, workgroup).
__global__ __launch_bounds__(kHeadWaves * 64, 1) void head_tile_kernel(
    const uint16_t* __restrict__ h, int H, const uint16_t* __restrict__ w, int V,
    int32_t mask_id, int tok0, int ntok, float* __restrict__ pm, float* __restrict__ ps,
    int32_t* __restrict__ pa) {
  extern __shared__ __align__(16) unsigned char head_smem[];
  const int HP = H + kHeadPad;
  uint16_t* hs = reinterpret_cast<uint16_t*>(head_smem);
  SoftStat* red = reinterpret_cast<SoftStat*>(head_smem + sizeof(uint16_t) * kHeadTokChunk * HP);

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;

  const long NG = (V + 15) / 16;
  const long NW = static_cast<long>(gridDim.x) * kHeadWaves;
  const long wid = static_cast<long>(blockIdx.x) * kHeadWaves + wave;
  const int g0 = static_cast<int>(wid * NG / NW);
  const int g1 = static_cast<int>((wid + 1) * NG / NW);
  const int KS = H / 32;
  const int nb = (KS + kHeadUnroll - 1) / kHeadUnroll;          // k-batches per chunk
  const int nchunks = (g1 - g0 + kHeadGroups - 1) / kHeadGroups;
  const int iters = nchunks * nb;

  // first batch in flight before the staging barrier
  u32x4 bcur[kHeadUnroll][kHeadGroups];
  if (iters > 0) {
    const int nq = (g1 - g0) < kHeadGroups ? (g1 - g0) : kHeadGroups;
    head_load_batch(bcur, w, V, H, g0, nq, 0, KS, c, g);
  }

  // stage this pass's hidden rows (rows >= ntok are zero)
  const int c8n = H / 8;
  for (int idx = tid; idx < kHeadTokChunk * c8n; idx += blockDim.x) {
    const int r = idx / c8n;
    const int c8 = idx - r * c8n;
    const u32x4 v = (r < ntok) ? ld16(h + static_cast<size_t>(tok0 + r) * H + c8 * 8)
                               : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(hs + r * HP + c8 * 8) = v;
  }
  __syncthreads();

  const bool two = ntok > 16;
  const uint16_t* arow0 = hs + c * HP + g * 8;
  const uint16_t* arow1 = hs + (16 + c) * HP + g * 8;

  SoftStat st[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) st[mt][i] = softstat_empty();

  f32x4 acc[kHeadGroups][2];
#pragma unroll
  for (int q = 0; q < kHeadGroups; ++q)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < iters; ++it) {
    const int chunk = it / nb;
    const int kb = it - chunk * nb;
    const int gb = g0 + chunk * kHeadGroups;
    const int nq = (g1 - gb) < kHeadGroups ? (g1 - gb) : kHeadGroups;   // wave-uniform
    const int s0 = kb * kHeadUnroll;

    u32x4 bnxt[kHeadUnroll][kHeadGroups];
    if (BDM_HEAD_PREFETCH && it + 1 < iters) {
      const int chunk1 = (it + 1) / nb;
      const int gb1 = g0 + chunk1 * kHeadGroups;
      const int nq1 = (g1 - gb1) < kHeadGroups ? (g1 - gb1) : kHeadGroups;
      head_load_batch(bnxt, w, V, H, gb1, nq1, ((it + 1) - chunk1 * nb) * kHeadUnroll, KS, c, g);
    }
#pragma unroll
    for (int u = 0; u < kHeadUnroll; ++u) {
      if (s0 + u < KS) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(arow0 + (s0 + u) * 32);
        const u32x4 a1 = two ? *reinterpret_cast<const u32x4*>(arow1 + (s0 + u) * 32)
                             : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < kHeadGroups; ++q) {
          acc[q][0] = mfma_bf16(a0, bcur[u][q], acc[q][0]);
          if (two) acc[q][1] = mfma_bf16(a1, bcur[u][q], acc[q][1]);
        }
      }
    }

    if (kb == nb - 1) {
      // online softmax over this chunk's columns (increasing vocabulary id per
      // lane, so a strict '>' keeps the lowest id among equal maxima)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          SoftStat& s = st[mt][i];
#pragma unroll
          for (int q = 0; q < kHeadGroups; ++q) {
            const int v = (gb + q) * 16 + c;
            if (q < nq && v < V && v != mask_id) {
              const float l = acc[q][mt][i];
              if (l > s.m) {
                s.s = (s.m == -INFINITY ? 0.0f : s.s * expf(s.m - l)) + 1.0f;
                s.m = l;
                s.a = v;
              } else {
                s.s += expf(l - s.m);
              }
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kHeadGroups; ++q)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (BDM_HEAD_PREFETCH) {
#pragma unroll
      for (int u = 0; u < kHeadUnroll; ++u)
#pragma unroll
        for (int q = 0; q < kHeadGroups; ++q) bcur[u][q] = bnxt[u][q];
    } else if (it + 1 < iters) {
      const int chunk1 = (it + 1) / nb;
      const int gb1 = g0 + chunk1 * kHeadGroups;
      const int nq1 = (g1 - gb1) < kHeadGroups ? (g1 - gb1) : kHeadGroups;
      head_load_batch(bcur, w, V, H, gb1, nq1, ((it + 1) - chunk1 * nb) * kHeadUnroll, KS, c, g);
    }
  }

  // merge the 16 lanes that share a row group, then the waves (fixed order)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const SoftStat s = row_merge_stat(st[mt][i]);
      if (c == 0) red[wave * kHeadTokChunk + mt * 16 + 4 * g + i] = s;
    }
  }
  __syncthreads();
  if (tid < ntok) {
    SoftStat s = red[tid];
    for (int wv = 1; wv < kHeadWaves; ++wv) s = softstat_merge(s, red[wv * kHeadTokChunk + tid]);
    const size_t o = static_cast<size_t>(tok0 + tid) * gridDim.x + blockIdx.x;
    pm[o] = s.m;
    ps[o] = s.s;
    pa[o] = s.a;
  }
}

// One workgroup.  16 threads (one DPP row) per token merge that token's
// partials (all loads issued first), the row reduction finishes the merge,
// and one wave applies the commit rule over the block.
__global__ __launch_bounds__(1024) void head_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const int32_t* __restrict__ pa,
    int T, int nparts, int32_t mask_id, float threshold, int fallback, int32_t* tokens,
    int32_t* __restrict__ argmax_out, float* __restrict__ conf_out,
    int32_t* __restrict__ n_committed) {
  extern __shared__ float smem[];
  float* sconf = smem;                                   // [T]
  int* sarg = reinterpret_cast<int*>(smem + T);         // [T]
  int* stok = sarg + T;                                  // [T]
  const int tid = threadIdx.x;
  for (int t = tid; t < T; t += blockDim.x) stok[t] = tokens[t];

  const int sub = tid & 15;          // thread within the token's row
  for (int t0 = 0; t0 < T; t0 += blockDim.x >> 4) {
    const int t = t0 + (tid >> 4);
    const bool on = t < T;           // row-uniform
    const size_t base = static_cast<size_t>(on ? t : 0) * nparts;
    SoftStat st = softstat_empty();
    for (int i0 = 0; i0 < nparts; i0 += 16 * 16) {
      SoftStat part[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 16 + sub;
        part[u] = (on && i < nparts) ? SoftStat{pm[base + i], ps[base + i], pa[base + i]}
                                     : softstat_empty();
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) st = softstat_merge(st, part[u]);
    }
    st = row_merge_stat(st);
    if (on && sub == 0) {
      const float cf = 1.0f / st.s;
      sconf[t] = cf;
      sarg[t] = st.a;
      if (argmax_out) argmax_out[t] = st.a;
      if (conf_out) conf_out[t] = cf;
    }
  }
  __syncthreads();
  if (tid >= kWave) return;

  // Commit rule, one wave.  Best masked row for the fallback: largest conf,
  // equal -> lowest position.
  const int lane = tid;
  int ncommit = 0;
  float best_c = -INFINITY;
  int best_t = INT32_MAX;
  for (int t0 = 0; t0 < T; t0 += kWave) {
    const int t = t0 + lane;
    int commit = 0;
    if (t < T && stok[t] == mask_id) {
      const float cf = sconf[t];
      if (cf >= threshold) commit = 1;
      if (cf > best_c || (cf == best_c && t < best_t)) {
        best_c = cf;
        best_t = t;
      }
    }
    if (commit) tokens[t] = sarg[t];
    ncommit += wave_sum_i(commit);
  }
  wave_argmax(best_c, best_t);
  if (fallback && ncommit == 0 && best_t != INT32_MAX) {
    if (lane == 0) tokens[best_t] = sarg[best_t];
    ncommit = 1;
  }
  if (lane == 0 && n_committed) *n_committed = ncommit;
}

void launch_head(const uint16_t* h, int T, int H, const uint16_t* w, int V, int32_t mask_id,
                 float threshold, int fallback, int32_t* tokens, int32_t* argmax, float* conf,
                 int32_t* n_committed, const HeadParts& parts, hipStream_t s) {
  const int grid = parts.grid;
  const size_t lds = head_lds_bytes(H);
  for (int t0 = 0; t0 < T; t0 += kHeadTokChunk) {
    const int n = (T - t0) < kHeadTokChunk ? (T - t0) : kHeadTokChunk;
    head_tile_kernel<<<grid, kHeadWaves * 64, lds, s>>>(h, H, w, V, mask_id, t0, n, parts.m,
                                                       parts.s, parts.a);
  }
  head_merge_kernel<<<1, 1024, static_cast<size_t>(T) * 12, s>>>(
      parts.m, parts.s, parts.a, T, grid, mask_id, threshold, fallback, tokens, argmax, conf,
      n_committed);
}

int head_prepare() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&head_tile_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(head_lds_bytes(BDM_MAX_HIDDEN))) == hipSuccess
             ? 0
             : -1;
}

}  // namespace bdm
