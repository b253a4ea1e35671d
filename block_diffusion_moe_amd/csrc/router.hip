// Router and top-k selection for the routed MoE layer.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": 256 routed experts, 8 picked
// per token, and a shared expert that every token uses.
//
//   router_kernel  logits l[t][e] = x_t . w_router[e] (+ bias[e]) in fp32.
//                  A small GEMM (T x H) . (H x E) on bf16 MFMA: each fp32
//                  router weight is split exactly into three bf16 terms
//                  (hi + mid + lo == w), so x . w is the fp32-accumulated sum
//                  of exact products, as an fp32 dot product would be.
//                  Workgroup tile: 16 experts x 32 tokens x one of 4 K-parts
//                  (4 waves split the part, every load issued first); the
//                  parts are summed in order by the select step.
//   select_kernel  per token (one wave each): the k largest logits (a
//                  ballot threshold search, equal logits -> lower id) and
//                  their softmax weights, renormalised over the picks; then
//                  the picks are grouped by expert (slot table + pair rows)
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
#ifndef BDM_RT_WIDE_TILES
#define BDM_RT_WIDE_TILES 4
#endif
constexpr int kRtWideTiles = BDM_RT_WIDE_TILES;   // token tiles per router workgroup, many blocks
#ifndef BDM_RT_WIDE_MIN_T
#define BDM_RT_WIDE_MIN_T 512
#endif
constexpr int kRtWideMinT = BDM_RT_WIDE_MIN_T;
constexpr int kRtMaxKs = 4;     // k-steps per wave: H <= kRouterParts * 4 * 4 * 32 = 2048

// Partial logits over one K-part: part[z][t][e] = sum_{h in part z} x[t][h] w[e][h].
// The fp32 partials are summed (in part order) with the bias by the select
// step.
// NTT token tiles of 32 per workgroup share one load and split of the
// router weights (NTT > 1 for many-block calls).
// NORM (NTT = 1): x is the layer's un-normalised input.  The workgroup takes
// the RMSNorm scale of each of its 32 rows with the arithmetic of the
// RMSNorm kernel (its 256 threads hold a row's 8-element chunks in the same
// order; the same summation tree, eps 1e-6), routes on bf16(x * scale), and
// the workgroups of expert tile 0 write those rows, bit for bit what the
// RMSNorm kernel writes, to xn (the experts' input).  Every workgroup reads
// and reduces all 32 rows (128 KB at H = 2048), which costs about what the
// separate RMSNorm launch does.
template <int NTT, bool NORM = false>
__global__ __launch_bounds__(kRtWaves * 64) void router_kernel(const uint16_t* __restrict__ x,
                                                              int T, int H,
                                                              const float* __restrict__ wr, int E,
                                                              float* __restrict__ part,
                                                              uint16_t* __restrict__ xn) {
  static_assert(!NORM || NTT == 1, "the fused RMSNorm covers one token tile");
  static_assert(kRtWaves * 64 == 256, "the RMSNorm chunk map needs 256 threads");
  __shared__ f32x4 red[2][kRtWaves][2][kWave];
  // NORM: per-thread sums of squares [thread][row] (row pitch 33: the
  // column reads below are conflict-free), the 32-thread partials and the
  // row scales
  __shared__ float rss[NORM ? 256 * 33 : 1];
  __shared__ float rq[NORM ? 8 * 32 : 1];
  __shared__ float rscale[NORM ? 32 : 1];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  // NORM: the scales of this lane's rows t0 + c and t0 + 16 + c
  float rsc0 = 1.0f, rsc1 = 1.0f;
  // NORM: this thread's 8-element chunk of each of the 32 rows, requested
  // before the router weights and the K-slice (in-order completion: the sums
  // below wait for these rows only)
  u32x4 raw[NORM ? 32 : 1];
  if constexpr (NORM) {
    const int tt0 = blockIdx.y * 32;
    const int i0 = threadIdx.x * 8;
    const bool on = i0 < H;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int row = tt0 + r;
      const bool ok = on && row < T;
      const u32x4 v = ld16(x + static_cast<size_t>(ok ? row : 0) * H + (on ? i0 : 0));
      raw[r] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // 16 bytes of a row times its scale, rounded as the RMSNorm kernel rounds
  auto norm16 = [](u32x4 v, float r) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __uint_as_float(v[j] << 16) * r;
      const float b = __uint_as_float(v[j] & 0xffff0000u) * r;
      o[j] = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    }
    return o;
  };
  const int e0 = blockIdx.x * 16;
  const int z = blockIdx.z;
  const int KS = H / 32;
  const int ksp = (KS + kRouterParts - 1) / kRouterParts;       // k-steps of this part
  const int ksw = (ksp + kRtWaves - 1) / kRtWaves;
  const int s0 = z * ksp + wave * ksw;
  const int s1 = min(min(s0 + ksw, (z + 1) * ksp), KS);

  const int er = (e0 + c) < E ? (e0 + c) : (E - 1);
  const float* wrow = wr + static_cast<size_t>(er) * H + g * 8;
  auto xload = [&](int t0, u32x4(&a0)[kRtMaxKs], u32x4(&a1)[kRtMaxKs]) {
    const bool ok0 = (t0 + c) < T, ok1 = (t0 + 16 + c) < T;
    const uint16_t* x0 = x + static_cast<size_t>(ok0 ? t0 + c : 0) * H + g * 8;
    const uint16_t* x1 = x + static_cast<size_t>(ok1 ? t0 + 16 + c : 0) * H + g * 8;
#pragma unroll
    for (int q = 0; q < kRtMaxKs; ++q) {
      const int s = (s0 + q < s1) ? s0 + q : 0;
      const u32x4 v0 = ld16(x0 + s * 32), v1 = ld16(x1 + s * 32);
      a0[q] = ok0 ? v0 : u32x4{0u, 0u, 0u, 0u};
      a1[q] = ok1 ? v1 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // NORM: scale the K-slice of rows t0 + c and t0 + 16 + c; expert tile 0
  // writes the normalised rows (each (row, k-step) once)
  auto xnorm = [&](int t0, u32x4(&a0)[kRtMaxKs], u32x4(&a1)[kRtMaxKs]) {
    const bool ok0 = (t0 + c) < T, ok1 = (t0 + 16 + c) < T;
#pragma unroll
    for (int q = 0; q < kRtMaxKs; ++q) {
      a0[q] = norm16(a0[q], rsc0);
      a1[q] = norm16(a1[q], rsc1);
      if (blockIdx.x == 0 && s0 + q < s1) {
        const int s = s0 + q;
        if (ok0)
          *reinterpret_cast<u32x4*>(xn + static_cast<size_t>(t0 + c) * H + s * 32 + g * 8) = a0[q];
        if (ok1)
          *reinterpret_cast<u32x4*>(xn + static_cast<size_t>(t0 + 16 + c) * H + s * 32 + g * 8) =
              a1[q];
      }
    }
  };

  // every load of this wave's K-slice first (clamped, no branches), then math
  float4 wa[kRtMaxKs], wb[kRtMaxKs];
  u32x4 a0[kRtMaxKs], a1[kRtMaxKs];
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    const int s = (s0 + q < s1) ? s0 + q : 0;
    wa[q] = *reinterpret_cast<const float4*>(wrow + s * 32);
    wb[q] = *reinterpret_cast<const float4*>(wrow + s * 32 + 4);
  }
  xload(blockIdx.y * NTT * 32, a0, a1);
  if constexpr (NORM) {
    // each row's sum of squares, the RMSNorm kernel's summation tree: per
    // thread fmaf over its 8 values in order, then a balanced binary tree
    // over the 256 threads in thread order (its DPP steps, rows of 16
    // lanes, the wave's 4 rows and the 4 waves pairwise are exactly that
    // tree).  Here the 32 rows are reduced side by side: thread (part p =
    // tid / 32, row r = tid % 32) sums threads 32p .. 32p + 31 of row r as a
    // 5-level tree, thread r < 32 the 8 parts as a 3-level one.
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(raw[r][j] << 16);
        const float hi = __uint_as_float(raw[r][j] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      rss[threadIdx.x * 33 + r] = ss;
    }
    __syncthreads();
    {
      const int r = threadIdx.x % 32, p = threadIdx.x / 32;
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = rss[(32 * p + j) * 33 + r];
#pragma unroll
      for (int w = 1; w < 32; w *= 2)
#pragma unroll
        for (int j = 0; j < 32; j += 2 * w) v[j] = v[j] + v[j + w];
      rq[p * 32 + r] = v[0];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      const int r = threadIdx.x;
      const float tot = ((rq[r] + rq[32 + r]) + (rq[64 + r] + rq[96 + r])) +
                        ((rq[128 + r] + rq[160 + r]) + (rq[192 + r] + rq[224 + r]));
      rscale[r] = 1.0f / sqrtf(tot / static_cast<float>(H) + 1e-6f);
    }
    __syncthreads();
    rsc0 = rscale[c];
    rsc1 = rscale[16 + c];
    xnorm(blockIdx.y * NTT * 32, a0, a1);
  }
  u32x4 bh[kRtMaxKs], bm[kRtMaxKs], bl[kRtMaxKs];
#pragma unroll
  for (int q = 0; q < kRtMaxKs; ++q) {
    const float wv[8] = {wa[q].x, wa[q].y, wa[q].z, wa[q].w, wb[q].x, wb[q].y, wb[q].z, wb[q].w};
    uint16_t hi[8], mi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split3(wv[j], hi[j], mi[j], lo[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bh[q][j] = static_cast<uint32_t>(hi[2 * j]) | (static_cast<uint32_t>(hi[2 * j + 1]) << 16);
      bm[q][j] = static_cast<uint32_t>(mi[2 * j]) | (static_cast<uint32_t>(mi[2 * j + 1]) << 16);
      bl[q][j] = static_cast<uint32_t>(lo[2 * j]) | (static_cast<uint32_t>(lo[2 * j + 1]) << 16);
    }
  }
  for (int tt = 0; tt < NTT; ++tt) {
    const int t0 = (blockIdx.y * NTT + tt) * 32;
    if (t0 >= T) break;                                  // workgroup-uniform
    const bool two = (t0 + 16) < T;
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kRtMaxKs; ++q) {
      if (s0 + q < s1) {
        acc0 = mfma_bf16(a0[q], bh[q], acc0);
        acc0 = mfma_bf16(a0[q], bm[q], acc0);
        acc0 = mfma_bf16(a0[q], bl[q], acc0);
        if (two) {
          acc1 = mfma_bf16(a1[q], bh[q], acc1);
          acc1 = mfma_bf16(a1[q], bm[q], acc1);
          acc1 = mfma_bf16(a1[q], bl[q], acc1);
        }
      }
    }
    if (tt + 1 < NTT && t0 + 32 < T) xload(t0 + 32, a0, a1);   // next tile in flight
    red[tt & 1][wave][0][lane] = acc0;
    red[tt & 1][wave][1][lane] = acc1;
    __syncthreads();
    if (threadIdx.x < 2 * kWave) {
      const int mt = threadIdx.x / kWave;
      const int ln = threadIdx.x % kWave;
      f32x4 sum = red[tt & 1][0][mt][ln];
#pragma unroll
      for (int w = 1; w < kRtWaves; ++w) sum += red[tt & 1][w][mt][ln];
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
}

// Order-preserving map of an fp32 logit to uint32 (larger float -> larger
// key); -0 is taken as +0 so that equal logits get equal keys.
__device__ __forceinline__ uint32_t logit_key(float l) {
  const uint32_t u = __float_as_uint(l);
  return (l == 0.0f) ? 0x80000000u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
}
__device__ __forceinline__ float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// One token's logit row, PER values per lane (expert lane + 64*i): the
// K-part partials summed in part order, plus the bias; past E and NaN -> -inf.
template <int PER>
__device__ __forceinline__ void load_logits(const float* __restrict__ part, size_t zstride,
                                            const float* __restrict__ bias, int E, int lane,
                                            float (&v)[PER]) {
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const int ec = e < E ? e : 0;
    float l = part[ec];
#pragma unroll
    for (int z = 1; z < kRouterParts; ++z) l += part[z * zstride + ec];
    if (bias) l += bias[ec];
    l = (e < E) ? l : -INFINITY;
    v[i] = (l == l) ? l : -INFINITY;              // NaN logits rank last
  }
}

// Top-k of one logit row.  The kc-th largest key (kc >= k candidates) is
// found bit by bit from the top with wave ballots (count of keys at or above
// a candidate), stopping early once exactly kc keys lie at or above it; the
// candidates are the keys above that threshold plus, among keys equal to it,
// the lowest expert ids.  They are gathered into lanes 0..kc-1 (ds_permute),
// ranked there (larger logit first, equal -> lower id) and moved to the lane
// of their rank, so lanes 0..k-1 hold the k picks.  Returns the j-th
// candidate in lane j (j < kc; its logit in *sel_l when asked) and, for
// j < k, the pick's weight (and probability over all E, WANT_P).
template <int PER, bool WANT_P = false>
__device__ __forceinline__ void topk_pick(const float (&v)[PER], int E, int k, int renorm,
                                          int lane, int& sel_e, float& sel_w,
                                          float* sel_p = nullptr, int kc = 0,
                                          float* sel_l = nullptr) {
  if (kc < k) kc = k;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = (lane + kWave * i < E) ? logit_key(v[i]) : 0u;
  // threshold search (every count is wave-uniform)
  uint32_t pre = 0u;
  bool exact = false;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = pre | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= kc) pre = cand;
    if (cnt == kc) {
      exact = true;
      break;
    }
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned long long pm[PER];
  int need = kc;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    pm[i] = __ballot(exact ? key[i] >= pre : key[i] > pre);
    need -= __popcll(pm[i]);
  }
  if (!exact) {
    // ties at the threshold: the lowest ids, in (i, lane) order
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const unsigned long long em = __ballot(key[i] == pre);
      const int take = min(need, __popcll(em));
      const bool mine = ((em >> lane) & 1ull) && __popcll(em & below) < take;
      pm[i] |= __ballot(mine);
      need -= take;
    }
  }
  // gather: the pick with compact index j goes to lane j (non-picks are
  // pushed to lane 63, which is never read: kc <= 32)
  int ck = 0, ce = 0, base = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n_i = __popcll(pm[i]);
    const int dst = ((pm[i] >> lane) & 1ull) ? base + __popcll(pm[i] & below) : kWave - 1;
    const int rk = __builtin_amdgcn_ds_permute(dst * 4, static_cast<int>(key[i]));
    const int re = __builtin_amdgcn_ds_permute(dst * 4, lane + kWave * i);
    if (lane >= base && lane < base + n_i) {
      ck = rk;
      ce = re;
    }
    base += n_i;
  }
  // rank among the kc candidates, then move each to the lane of its rank
  int rank = 0;
  for (int q = 0; q < kc; ++q) {
    const uint32_t kq = static_cast<uint32_t>(__builtin_amdgcn_readlane(ck, q));
    const int eq = __builtin_amdgcn_readlane(ce, q);
    rank += (kq > static_cast<uint32_t>(ck) || (kq == static_cast<uint32_t>(ck) && eq < ce)) ? 1
                                                                                          : 0;
  }
  const int dst = lane < kc ? rank : kWave - 1;
  const int sk = __builtin_amdgcn_ds_permute(dst * 4, ck);
  const int se = __builtin_amdgcn_ds_permute(dst * 4, ce);
  if (sel_l) *sel_l = (lane < kc) ? key_logit(static_cast<uint32_t>(sk)) : -INFINITY;
  const float sel_v = (lane < k) ? key_logit(static_cast<uint32_t>(sk)) : -INFINITY;
  sel_e = (lane < kc) ? se : 0;
  const float first_v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
  // w_j = exp(l_j - l_max) / (sum over the picks when renormalised, else over
  // all E); p_j (WANT_P) = exp(l_j - l_max) / sum over all E
  const float z = (lane < k) ? expf(sel_v - first_v) : 0.0f;
  float den_all = 0.0f;
  if (WANT_P || !renorm) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      if (e < E) s += expf(v[i] - first_v);
    }
    den_all = wave_sum(s);
  }
  sel_w = z / (renorm ? wave_sum(z) : den_all);
  if (WANT_P) *sel_p = z / den_all;
}

constexpr int kSelWaves = 4;       // tokens per select workgroup (one wave each)
constexpr int kSelOneWaves = 16;   // waves of the single-workgroup select (small blocks)
constexpr int kSelOneMaxT = 16;    // largest block the single-workgroup select takes

// Group the T*k picks by expert for the expert kernels (every thread of the
// workgroup calls this; picks in LDS or global memory, -1 = no expert):
//   slots[i] = {expert, offset, count, 0}: one work item of at most
//              kSlotChunk tokens of a group -- the shared expert's chunks
//              (group E, all T tokens) first, then the chunks of routed
//              experts with at least 16 tokens, then the others, experts in
//              increasing id and an expert's chunks consecutive -- and
//              {-1, 0, 0, 0} for i = n .. moe_max_slots - 1;
//   pair_rows[offset .. offset+count) = the (token, slot) rows t*(k+1)+j of
//              the chunk's tokens (shared: t*(k+1)+k); the groups' ranges
//              follow expert id order after the shared expert's [0, T).
// Wave 0 ranks the experts: lane L holds experts L*epl .. L*epl+epl-1, so
// (lane, j) order is id order, and ballot popcounts (light experts: one
// slot each) and bit-sliced ballot prefixes (heavy experts' chunk counts,
// pair offsets) give every expert's first slot and pair offset.  The order
// inside a group is whatever the LDS atomics produce; every row's result is
// computed on its own, so outputs do not depend on it.
template <int PER>
__device__ void group_picks(const int32_t* picks, int T, int E, int k, int has_shared, int* cnt,
                            int* eoff, int* fill, int4* __restrict__ slots,
                            int32_t* __restrict__ pair_rows, int32_t* __restrict__ info) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int K1 = k + 1;
  for (int e = tid; e <= E; e += blockDim.x) {
    cnt[e] = (e == E) ? (has_shared ? T : 0) : 0;
    fill[e] = 0;
  }
  __syncthreads();
  // picks in batches of 8 per thread, every load of a batch issued first
  const int np = T * k;
  for (int p0 = 0; p0 < np; p0 += 8 * static_cast<int>(blockDim.x)) {
    int eb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * static_cast<int>(blockDim.x) + tid;
      eb[u] = p < np ? picks[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (eb[u] >= 0 && eb[u] < E) atomicAdd(&cnt[eb[u]], 1);
      else if (eb[u] != -1) note_oob(kChkExpert);   // -1: an empty pick
    }
  }
  __syncthreads();
  const int nsh = has_shared ? (T + kSlotChunk - 1) / kSlotChunk : 0;   // shared chunks
  const int nslot = moe_max_slots(T, E, k, has_shared);                // slots[] extent
  if (wave == 0) {
    constexpr int EPL = PER;                          // experts per lane, at most
    const int epl = (E + kWave - 1) / kWave;          // E <= 64 * PER
    const unsigned long long bel = (1ull << lane) - 1ull;
    int c[EPL];
    int nl = 0, lb = 0;              // light experts: total, in lanes below
    int hch = 0, tot = 0;            // this lane's heavy chunks and pairs
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane * epl + j;
      c[j] = (j < epl && e < E) ? cnt[e] : 0;
      const unsigned long long ml = __ballot(c[j] > 0 && c[j] < 16);
      nl += __popcll(ml);
      lb += __popcll(ml & bel);
      if (c[j] >= 16) hch += (c[j] + kSlotChunk - 1) / kSlotChunk;
      tot += c[j];
    }
    // exclusive prefixes over the lanes, one ballot per bit (a lane's pairs
    // are < 2^16: at most T <= 2^11 per expert, PER <= 16 experts; its
    // chunks fewer still)
    int hb = 0, nh = 0;
    int pref = has_shared ? T : 0;
#pragma unroll
    for (int bit = 0; bit < 16; ++bit) {
      const unsigned long long bh = __ballot((hch >> bit) & 1);
      hb += __popcll(bh & bel) << bit;
      nh += __popcll(bh) << bit;
      pref += __popcll(__ballot((tot >> bit) & 1) & bel) << bit;
    }
    int ho = 0, lo = 0;                       // this lane's slots so far
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if (c[j] > 0) {
        const int e = lane * epl + j;
        if (c[j] >= 16) {
          const int pos = nsh + hb + ho;
          const int nch = (c[j] + kSlotChunk - 1) / kSlotChunk;
          int q = 0;
          for (int o = 0; o < c[j]; o += kSlotChunk, ++q) {
            const int m = c[j] - o < kSlotChunk ? c[j] - o : kSlotChunk;
            slots[chk(pos + q, nslot, kChkWs)] = int4{e, pref + o, m, nch};
          }
          ho += q;
        } else {
          slots[chk(nsh + nh + lb + lo, nslot, kChkWs)] = int4{e, pref, c[j], 1};
          ++lo;
        }
        eoff[e] = pref;
      }
      pref += c[j];
    }
    const int n = nsh + nh + nl;
    for (int i = lane; i < nsh; i += kWave) {
      const int o = i * kSlotChunk;
      slots[i] = int4{E, o, T - o < kSlotChunk ? T - o : kSlotChunk, nsh};
    }
    for (int i = n + lane; i < nslot; i += kWave) slots[i] = int4{-1, 0, 0, 0};
    if (lane == 0) info[0] = n;
  }
  // scatter the pairs
  __syncthreads();
  for (int p0 = 0; p0 < np; p0 += 8 * static_cast<int>(blockDim.x)) {
    int eb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * static_cast<int>(blockDim.x) + tid;
      eb[u] = p < np ? picks[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = eb[u];
      if (e < 0 || e >= E) continue;
      const int p = p0 + u * static_cast<int>(blockDim.x) + tid;
      const int tt = p / k;
      pair_rows[chk(eoff[e] + atomicAdd(&fill[e], 1), T * K1, kChkPairRow)] =
          tt * K1 + (p - tt * k);
    }
  }
  if (has_shared)
    for (int tt = tid; tt < T; tt += blockDim.x) pair_rows[tt] = tt * K1 + k;
}

// Top-k of every token.  SINGLE (T <= 16): one workgroup of NW waves takes
// every token (wave w: token w), keeps the picks in LDS and groups them
// itself.  Otherwise one wave per token, NW tokens per workgroup, and
// group_kernel follows (a completion ticket instead would need a
// device-wide release in every workgroup, its L2 written back, which costs
// more than the second launch).  FIRST (first pass of the block coreset
// selector): the picks, their weights and their probabilities over all E
// (topk_p) only.
template <int PER, int NW, bool SINGLE, bool FIRST>
__global__ __launch_bounds__(NW * 64) void select_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int T, int E, int k,
    int renorm, int has_shared, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ topk_p, int32_t* __restrict__ cand_id, float* __restrict__ cand_l,
    int4* __restrict__ slots, int32_t* __restrict__ pair_rows,
    int32_t* __restrict__ info, int32_t* __restrict__ user_idx, float* __restrict__ user_w) {
  constexpr bool kGroups = SINGLE && !FIRST;
  __shared__ int cnt[kGroups ? BDM_MAX_EXPERTS + 1 : 1];
  __shared__ int eoff[kGroups ? BDM_MAX_EXPERTS + 1 : 1];
  __shared__ int fill[kGroups ? BDM_MAX_EXPERTS + 1 : 1];
  __shared__ int spick[SINGLE ? kSelOneMaxT * BDM_MAX_TOPK : 1];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  const int t = SINGLE ? wave : blockIdx.x * NW + wave;
  if (t < T) {
    float v[PER];
    load_logits<PER>(part + static_cast<size_t>(t) * E, static_cast<size_t>(T) * E, bias, E,
                     lane, v);
    int sel_e;
    float sel_w, sel_p, sel_l;
    // the first pass of the coreset selector also ranks the next candidates:
    // a token's re-route over the kept experts takes them in this order
    const int kc = FIRST ? (E < kCoreCand ? E : kCoreCand) : k;
    topk_pick<PER, FIRST>(v, E, k, renorm, lane, sel_e, sel_w, &sel_p, kc, &sel_l);
    if (FIRST && lane < kCoreCand) {
      cand_id[t * kCoreCand + lane] = lane < kc ? sel_e : -1;
      cand_l[t * kCoreCand + lane] = lane < kc ? sel_l : -INFINITY;
    }
    if (lane < k) {
      topk_idx[t * k + lane] = sel_e;
      topk_w[t * k + lane] = sel_w;
      if (FIRST) topk_p[t * k + lane] = sel_p;
      if (!FIRST && user_idx) user_idx[t * k + lane] = sel_e;
      if (!FIRST && user_w) user_w[t * k + lane] = sel_w;
      if (SINGLE) spick[t * k + lane] = sel_e;
    }
  }
  if constexpr (kGroups) {
    __syncthreads();
    group_picks<PER>(spick, T, E, k, has_shared, cnt, eoff, fill, slots, pair_rows, info);
  }
}

// The grouping after a multi-workgroup top-k (or coreset) kernel: one
// workgroup of 1024 threads.
template <int PER>
__global__ __launch_bounds__(1024) void group_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                     int E, int k, int has_shared,
                                                     int4* __restrict__ slots,
                                                     int32_t* __restrict__ pair_rows,
                                                     int32_t* __restrict__ info) {
  __shared__ int cnt[BDM_MAX_EXPERTS + 1];
  __shared__ int eoff[BDM_MAX_EXPERTS + 1];
  __shared__ int fill[BDM_MAX_EXPERTS + 1];
  group_picks<PER>(topk_idx, T, E, k, has_shared, cnt, eoff, fill, slots, pair_rows, info);
}

constexpr int kCsWaves = 16;       // waves of a coreset workgroup (one block of tokens)

// Re-route one token over the kept experts, given its first-pass picks (lane
// j < k holds pick j in `fe`, decreasing logit) and its logit row v.  The
// kept first-pass picks stay first, in their order (they are the token's
// largest logits); the remaining min(k, keep) - (kept first-pass picks)
// slots take the largest logits among kept experts that were not picked
// (wave argmax rounds, equal -> lower id).  Weights as in topk_pick over the
// kept experts.  Lane s < k returns slot s (-1 / 0 past min(k, keep)).
template <int PER>
__device__ __forceinline__ void reroute_pick(const float (&v)[PER], int fe, const int* rank_of,
                                             int keep, int E, int k, int renorm, int lane,
                                             int& sel_e, float& sel_w) {
  const unsigned long long below = (1ull << lane) - 1ull;
  const int fr = (lane < k && fe >= 0) ? rank_of[chk(fe, E, kChkExpert)] : -1;
  const bool fkeep = fr >= 0 && fr < keep;
  const unsigned long long km = __ballot(fkeep);
  const int nfk = __popcll(km);
  const int kk = min(k, keep);
  // which of this lane's experts are first-pass picks, which are kept
  uint32_t picked = 0u, allowed = 0u;
#pragma unroll
  for (int q = 0; q < BDM_MAX_TOPK; ++q) {
    if (q < k) {
      const int eq = __builtin_amdgcn_readlane(fe, q);
      if ((eq & (kWave - 1)) == lane) picked |= 1u << (eq / kWave);
    }
  }
  float cv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const int r = e < E ? rank_of[e] : -1;
    const bool ok = r >= 0 && r < keep;
    allowed |= (ok ? 1u : 0u) << i;
    cv[i] = (ok && !((picked >> i) & 1u)) ? v[i] : -INFINITY;
  }
  // the new picks: lane r (< nnew) receives the r-th one
  const int nnew = kk - nfk;
  int ne = -1;
  float nv = -INFINITY;
  for (int r = 0; r < nnew; ++r) {
    float bv = -INFINITY;
    int be = INT32_MAX;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      if (cv[i] > bv || (cv[i] == bv && cv[i] != -INFINITY && e < be)) {
        bv = cv[i];
        be = e;
      }
    }
    wave_argmax(bv, be);
    if (lane == r) {
      ne = be;
      nv = bv;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + kWave * i == be) cv[i] = -INFINITY;
  }
  // logit of this lane's first-pass pick (from the lane that holds it)
  const int src = (fe >= 0 ? fe : 0) & (kWave - 1);
  float fv = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float x = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(v[i])));
    if (fe >= 0 && fe / kWave == i) fv = x;
  }
  // slots: kept first-pass picks (pushed to their compact position), then
  // the new ones (pulled from lanes 0 .. nnew-1)
  const int dst = fkeep ? __popcll(km & below) : kWave - 1;
  const int pe = __builtin_amdgcn_ds_permute(dst * 4, fe);
  const float pv = __int_as_float(__builtin_amdgcn_ds_permute(dst * 4, __float_as_int(fv)));
  const int from = (lane >= nfk && lane < kk) ? lane - nfk : 0;
  const int qe = __builtin_amdgcn_ds_bpermute(from * 4, ne);
  const float qv = __int_as_float(__builtin_amdgcn_ds_bpermute(from * 4, __float_as_int(nv)));
  float sel_v = -INFINITY;
  sel_e = -1;
  if (lane < nfk) {
    sel_e = pe;
    sel_v = pv;
  } else if (lane < kk) {
    sel_e = qe;
    sel_v = qv;
  }
  const float first_v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
  const float z = (lane < kk) ? expf(sel_v - first_v) : 0.0f;
  float den;
  if (renorm) {
    den = wave_sum(z);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((allowed >> i) & 1u) s += expf(v[i] - first_v);
    den = wave_sum(s);
  }
  sel_w = (lane < kk) ? z / den : 0.0f;
}

// Block coreset expert selector, one workgroup per block of B <= 32 tokens
// (page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "The expert selection"):
//   first pass (select_kernel FIRST): every token's top-k, weights, the
//             picks' probabilities over all E, and its 32 best experts
//             ranked (the re-route's candidates);
//   mass_e  = sum over the block's tokens of the probabilities of the picks
//             of e (fp32; four partial sums over token ranges, added in a
//             fixed order);
//   order   = touched experts by mass, larger first (equal -> lower id);
//   kept    = the shortest prefix whose cumulative mass (fp32, fixed order)
//             reaches top_p times the total, at least one expert;
//   re-route: each token's top-min(k, |kept|) over the kept experts (the
//             others at -inf), weights as in the plain routing; the rest of
//             its k slots hold -1 and weight 0.
// The workgroup's 16 waves share one CU, so the kernel is bound by its VALU
// issue rate: the masses are a scatter of each token's picks (a token's
// picks are distinct experts: one token per step, its picks in parallel,
// tokens in order, the summation order of a per-expert loop over the
// picks), ranks are counted over the touched experts only, and a token's
// re-route takes the first min(k, |kept|) kept experts of its ranked
// candidates -- the kept first-pass picks in their order, then the best
// kept experts it did not pick, exactly what rounds of argmax over the kept
// experts give.  A token whose candidates hold too few kept experts (or any
// token when the weights are not renormalised, whose denominator needs the
// whole row) loads its logit row and takes the argmax rounds.
// Then the grouping: by the block's own workgroup when there is one block
// (GROUP), else by group_kernel launched after this kernel.
template <int PER, bool GROUP>
__global__ __launch_bounds__(kCsWaves * 64) void coreset_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int T, int E, int k,
    int renorm, float top_p, int B, int has_shared, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, const float* __restrict__ topk_p,
    const int32_t* __restrict__ cand_id, const float* __restrict__ cand_l,
    int4* __restrict__ slots, int32_t* __restrict__ pair_rows, int32_t* __restrict__ info,
    int32_t* __restrict__ user_idx, float* __restrict__ user_w, int32_t* __restrict__ n_kept) {
  constexpr int kParts = 4;                     // partial sums per expert mass
  __shared__ int cnt[BDM_MAX_EXPERTS + 1];
  __shared__ int eoff[BDM_MAX_EXPERTS + 1];
  __shared__ int fill[BDM_MAX_EXPERTS + 1];
  __shared__ float mpart[kParts][BDM_MAX_EXPERTS];
  __shared__ float smass[BDM_MAX_EXPERTS];      // masses in mass order
  __shared__ int rank_of[BDM_MAX_EXPERTS];      // position in mass order, -1 untouched
  __shared__ int tlist[BDM_MAX_EXPERTS];        // touched experts (any order) and masses
  __shared__ float tmass[BDM_MAX_EXPERTS];
  __shared__ int sidx[BDM_CORESET_MAX_BLOCK * BDM_MAX_TOPK];
  __shared__ float sp[BDM_CORESET_MAX_BLOCK * BDM_MAX_TOPK];
  __shared__ float sw[BDM_CORESET_MAX_BLOCK * BDM_MAX_TOPK];
  __shared__ int scid[BDM_CORESET_MAX_BLOCK * kCoreCand];
  __shared__ float scl[BDM_CORESET_MAX_BLOCK * kCoreCand];
  __shared__ int s_ntouch, s_nkeep;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int t0 = blockIdx.x * B;
  const int nb = min(B, T - t0);                // tokens of this block
  const int E16 = (E + 15) & ~15;
  const int nbk = nb * k;
  const int nbk16 = (nbk + 15) & ~15;
  const unsigned long long below = (1ull << lane) - 1ull;

  // the block's first-pass picks (padded with id -1 to a multiple of 16),
  // weights, probabilities and ranked candidates; zeroed partial masses
  for (int i = tid; i < nbk16; i += blockDim.x) {
    const bool in = i < nbk;
    sidx[i] = in ? topk_idx[t0 * k + i] : -1;
    sp[i] = in ? topk_p[t0 * k + i] : 0.0f;
    sw[i] = in ? topk_w[t0 * k + i] : 0.0f;
  }
  for (int i = tid; i < nb * kCoreCand; i += blockDim.x) {
    scid[i] = cand_id[t0 * kCoreCand + i];
    scl[i] = cand_l[t0 * kCoreCand + i];
  }
  for (int i = tid; i < kParts * BDM_MAX_EXPERTS; i += blockDim.x) mpart[0][i] = 0.0f;
  if (tid == 0) s_ntouch = 0;
  __syncthreads();
  // mass: part pp holds the picks [pp chunk, (pp + 1) chunk) (in token
  // order); wave pp adds them token by token, lane j taking a token's pick j
  // (distinct experts), so every partial sum runs over its picks in order
  const int nparts = (static_cast<int>(blockDim.x) / E16 >= kParts) ? kParts : 1;
  const int chunk = ((nbk16 / 16 + nparts - 1) / nparts) * 16;
  if (wave < nparts && lane < k) {
    const int i0 = wave * chunk;
    const int i1 = min(nbk, min(nbk16, i0 + chunk));
    // eight tokens' picks read first, then added in token order
    for (int tb = i0 / k; tb * k < i1; tb += 8) {
      int ee[8];
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = (tb + u) * k + lane;
        const bool in = i >= i0 && i < i1;
        ee[u] = in ? sidx[i] : -1;
        pv[u] = in ? sp[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (ee[u] >= 0 && ee[u] < E) mpart[wave][ee[u]] += pv[u];
        else if (ee[u] != -1) note_oob(kChkExpert);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    float m = mpart[0][e];
    for (int pp = 1; pp < nparts; ++pp) m += mpart[pp][e];
    cnt[e] = 0;
    rank_of[e] = -1;
    if (m > 0.0f) {
      const int q = chk(atomicAdd(&s_ntouch, 1), E, kChkCand);
      tlist[q] = e;
      tmass[q] = m;
    }
  }
  __syncthreads();
  // rank in mass order (larger first, equal -> lower id), counted over the
  // touched experts: every wave holds the whole list in registers (lane l:
  // entries l, l + 64, ...; a positive mass orders as its bits), wave w
  // ranks the 64 entries of group w % ng against the part w / ng of the
  // list, reading the other entries with readlane (no memory in the loop)
  const int nt = s_ntouch;
  {
    uint32_t kb[PER];
    int kid[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = lane + kWave * i;
      kb[i] = q < nt ? __float_as_uint(tmass[chk(q, E, kChkCand)]) : 0u;
      kid[i] = q < nt ? tlist[chk(q, E, kChkCand)] : INT32_MAX;
    }
    const int ng = (nt + kWave - 1) / kWave;               // groups of 64 entries
    const int nsp = ng > 0 ? max(1, kCsWaves / ng) : 1;   // parts of the list
    if (ng > 0 && wave < ng * nsp) {
      const int gq = wave % ng, pp = wave / ng;
      const int chunk = (nt + nsp - 1) / nsp;
      const int j0 = pp * chunk, j1 = min(nt, j0 + chunk);
      uint32_t mb = 0u;
      int me = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == gq) {
          mb = kb[i];
          me = kid[i];
        }
      int r = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int lo = max(j0 - kWave * i, 0), hi = min(j1 - kWave * i, kWave);
        for (int l = lo; l < hi; ++l) {
          const uint32_t bj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kb[i]), l));
          const int idj = __builtin_amdgcn_readlane(kid[i], l);
          r += (bj > mb || (bj == mb && idj < me)) ? 1 : 0;
        }
      }
      if (gq * kWave + lane < nt) atomicAdd(&cnt[chk(me, E, kChkExpert)], r);   // any order
    }
  }
  __syncthreads();
  for (int q = tid; q < nt; q += blockDim.x) {
    const int e = tlist[q];
    const int r = chk(cnt[e], E, kChkCand);
    smass[r] = tmass[q];
    rank_of[e] = r;
  }
  __syncthreads();
  // cumulative mass in order (lane L sums a contiguous chunk, then a fixed
  // scan over lanes) and the cut
  if (wave == 0) {
    const int per = (nt + kWave - 1) / kWave;
    const int i0 = lane * per;
    float loc = 0.0f;
    for (int i = i0; i < min(i0 + per, nt); ++i) loc += smass[i];
    float incl = loc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    const float total = __shfl(incl, kWave - 1, kWave);
    const float thr = top_p * total;
    const float up = __shfl_up(incl, 1, kWave);
    float cum = lane == 0 ? 0.0f : up;           // exclusive prefix of this chunk
    int below_n = 0;
    for (int i = i0; i < min(i0 + per, nt); ++i) {
      cum += smass[i];
      below_n += (cum < thr) ? 1 : 0;
    }
    below_n = wave_sum_i(below_n);
    if (lane == 0) {
      const int keep = min(max(below_n + 1, 1), nt);
      s_nkeep = keep;
      if (n_kept) n_kept[blockIdx.x] = keep;
    }
  }
  __syncthreads();
  // re-route every token of the block over the kept experts; a token whose
  // first-pass picks are all kept keeps them and (renormalised) their
  // weights, which is what the re-route would compute
  const int keep = s_nkeep;
  const int nc = E < kCoreCand ? E : kCoreCand;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int tl = wave + r * kCsWaves;
    if (tl < nb) {
      const int fe = lane < k ? sidx[tl * k + lane] : -1;
      const int fr = (lane < k && fe >= 0) ? rank_of[chk(fe, E, kChkExpert)] : -1;
      const bool fkeep = fr >= 0 && fr < keep;
      int sel_e;
      float sel_w;
      if (renorm && __popcll(__ballot(fkeep)) == k) {
        sel_e = fe;
        sel_w = lane < k ? sw[tl * k + lane] : 0.0f;
      } else {
        const int kk = min(k, keep);
        const int ce = lane < nc ? scid[tl * kCoreCand + lane] : -1;
        const float cl = lane < nc ? scl[tl * kCoreCand + lane] : -INFINITY;
        const bool ok = ce >= 0 && ce < E && cl != -INFINITY && rank_of[ce] >= 0 &&
                        rank_of[ce] < keep;
        const unsigned long long cm = __ballot(ok);
        if (renorm && __popcll(cm) >= kk) {
          // the first kk kept candidates, in rank order, to lanes 0 .. kk-1
          const int pos = __popcll(cm & below);
          const int dst = (ok && pos < kk) ? pos : kWave - 1;
          const int pe = __builtin_amdgcn_ds_permute(dst * 4, ce);
          const float pv =
              __int_as_float(__builtin_amdgcn_ds_permute(dst * 4, __float_as_int(cl)));
          const float sel_v = lane < kk ? pv : -INFINITY;
          sel_e = lane < kk ? pe : -1;
          const float first_v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
          const float z = (lane < kk) ? expf(sel_v - first_v) : 0.0f;
          const float den = wave_sum(z);
          sel_w = (lane < kk) ? z / den : 0.0f;
        } else {
          float v[PER];
          load_logits<PER>(part + static_cast<size_t>(t0 + tl) * E, static_cast<size_t>(T) * E,
                           bias, E, lane, v);
          reroute_pick<PER>(v, fe, rank_of, keep, E, k, renorm, lane, sel_e, sel_w);
        }
      }
      if (lane < k) {
        const int t = t0 + tl;
        topk_idx[t * k + lane] = sel_e;
        topk_w[t * k + lane] = sel_w;
        if (user_idx) user_idx[t * k + lane] = sel_e;
        if (user_w) user_w[t * k + lane] = sel_w;
        sidx[tl * k + lane] = sel_e;            // this wave's own entries only
      }
    }
  }
  if constexpr (GROUP) {                 // one block: its workgroup groups the picks
    __syncthreads();
    group_picks<PER>(sidx, T, E, k, has_shared, cnt, eoff, fill, slots, pair_rows, info);
  }
}

void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, float top_p, int block,
                   const MoeMeta& meta, int32_t* user_idx, float* user_w, int32_t* n_kept,
                   uint16_t* xn, hipStream_t s) {
  if (T >= kRtWideMinT) {
    // many tiles per workgroup: a separate RMSNorm when asked for
    if (xn) {
      launch_rmsnorm(x, nullptr, 1e-6f, T, H, xn, s);
      x = xn;
    }
    const dim3 grid((E + 15) / 16, (T + 32 * kRtWideTiles - 1) / (32 * kRtWideTiles),
                    kRouterParts);
    router_kernel<kRtWideTiles><<<grid, kRtWaves * 64, 0, s>>>(x, T, H, wr, E, meta.logits,
                                                               nullptr);
  } else {
    const dim3 grid((E + 15) / 16, (T + 31) / 32, kRouterParts);
    if (xn)
      router_kernel<1, true><<<grid, kRtWaves * 64, 0, s>>>(x, T, H, wr, E, meta.logits, xn);
    else
      router_kernel<1><<<grid, kRtWaves * 64, 0, s>>>(x, T, H, wr, E, meta.logits, nullptr);
  }
  const int nsel = (T + kSelWaves - 1) / kSelWaves;
  const bool core = top_p > 0.0f;
  const int ncs = core ? (T + block - 1) / block : 0;
#define BDM_SELECT(P)                                                                          \
  if (core) {                                                                                  \
    select_kernel<P, kSelWaves, false, true><<<nsel, kSelWaves * 64, 0, s>>>(                  \
        meta.logits, bias, T, E, k, renorm, has_shared, meta.topk_idx, meta.topk_w,            \
        meta.topk_p, meta.cand_id, meta.cand_l, meta.slots, meta.pair_rows, meta.info,         \
        user_idx, user_w);                                                                     \
    if (ncs > 1) {                                                                             \
      coreset_kernel<P, false><<<ncs, kCsWaves * 64, 0, s>>>(                                  \
          meta.logits, bias, T, E, k, renorm, top_p, block, has_shared, meta.topk_idx,         \
          meta.topk_w, meta.topk_p, meta.cand_id, meta.cand_l, meta.slots, meta.pair_rows,     \
          meta.info, user_idx, user_w, n_kept);                                                \
      group_kernel<P><<<1, 1024, 0, s>>>(meta.topk_idx, T, E, k, has_shared, meta.slots,       \
                                         meta.pair_rows, meta.info);                           \
    } else {                                                                                   \
      coreset_kernel<P, true><<<1, kCsWaves * 64, 0, s>>>(                                     \
          meta.logits, bias, T, E, k, renorm, top_p, block, has_shared, meta.topk_idx,         \
          meta.topk_w, meta.topk_p, meta.cand_id, meta.cand_l, meta.slots, meta.pair_rows,     \
          meta.info, user_idx, user_w, n_kept);                                                \
    }                                                                                          \
  } else if (T <= kSelOneMaxT) {                                                               \
    select_kernel<P, kSelOneWaves, true, false><<<1, kSelOneWaves * 64, 0, s>>>(               \
        meta.logits, bias, T, E, k, renorm, has_shared, meta.topk_idx, meta.topk_w,            \
        meta.topk_p, meta.cand_id, meta.cand_l, meta.slots, meta.pair_rows, meta.info,         \
        user_idx, user_w);                                                                     \
  } else {                                                                                     \
    select_kernel<P, kSelWaves, false, false><<<nsel, kSelWaves * 64, 0, s>>>(                 \
        meta.logits, bias, T, E, k, renorm, has_shared, meta.topk_idx, meta.topk_w,            \
        meta.topk_p, meta.cand_id, meta.cand_l, meta.slots, meta.pair_rows, meta.info,         \
        user_idx, user_w);                                                                     \
    group_kernel<P><<<1, 1024, 0, s>>>(meta.topk_idx, T, E, k, has_shared, meta.slots,         \
                                       meta.pair_rows, meta.info);                             \
  }
  if (E <= 256) {
    BDM_SELECT(4)
  } else if (E <= 512) {
    BDM_SELECT(8)
  } else {
    BDM_SELECT(16)
  }
#undef BDM_SELECT
}

BDM_DEBUG_WORD_READER(debug_words_router)

}  // namespace bdm
