// Untied output head fused with the low-confidence unmask rule.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": the head has its own
// 508,559,360 weights and every step streams all of them; section "How it
// writes", steps 2-3: each slot's prediction excludes the mask token and
// carries its probability; masked slots at or above the threshold are
// filled, and if none is, the best masked slot alone.
//
//   head_tile_kernel   persistent, one workgroup per CU.  The weight rows
//                      stream from HBM once into MFMA B registers; the block's
//                      hidden states (<= 32 rows per pass) sit in LDS as the
//                      A operand.  The logits never leave registers: each
//                      (token, workgroup) keeps only the online-softmax triple
//                      (max, sum of exp, argmax).
//   head_coop_kernel   the same with the 8 waves of a workgroup splitting K
//                      and moving in step (up to 64 rows per pass; the passes
//                      of more rows in one launch).
//   head_gemm_kernel   from 256 rows: a tiled GEMM (256 x 256 tiles staged in
//                      LDS, the whole K per tile) with the same epilogue.
//   head_merge_kernel  one workgroup: merges the triples of all workgroups in
//                      a fixed tree per token -> conf = 1 / sum, argmax; then
//                      applies the commit rule and its progress fallback.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

#ifndef BDM_HEAD_QG
#define BDM_HEAD_QG 1
#endif
#ifndef BDM_HEAD_U
#define BDM_HEAD_U 8
#endif
constexpr int kHeadQG = BDM_HEAD_QG;   // 16-row vocabulary groups a wave multiplies together
constexpr int kHeadU = BDM_HEAD_U;     // k-steps per loaded batch
constexpr int kHeadPad = 8;            // bf16 padding per staged row (bank spread)

size_t head_lds_bytes(int H) {
  return static_cast<size_t>(kHeadTokChunk) * (H + kHeadPad) * sizeof(uint16_t) +
         static_cast<size_t>(kHeadWaves) * kHeadTokChunk * sizeof(SoftStat);
}

// Persistent: one workgroup per CU, 8 waves.  The <= 32 hidden rows of this
// pass are staged once in LDS (A operand).  The vocabulary is cut into
// chunks of QG 16-row groups and every wave of the grid takes one
// contiguous run of chunks (lengths differ by at most one), streaming those
// weight rows once from HBM as the B operand.  The loop runs over
// (chunk, k-batch) pairs; the next batch's loads are issued before the
// current batch's MFMAs, and no load sits behind a branch (rows past V are
// clamped to a valid row and dropped in the epilogue), so a wave always has
// a batch in flight, also across chunk boundaries.  Each lane keeps
// online-softmax state for its 8 (token, column) slots across the run; the
// per-wave results are merged across lanes and waves in a fixed order and
// written as one partial per (token, workgroup).  U = k-steps per batch.
template <int QG, int U, bool NBEVEN>
__global__ __launch_bounds__(kHeadWaves * 64, 1) void head_tile_kernel(
    const uint16_t* __restrict__ h, int H, const uint16_t* __restrict__ w, int V, int voff,
    int layout, int32_t mask_id, int tok0, int ntok, float* __restrict__ pm,
    float* __restrict__ ps, int32_t* __restrict__ pa, int pstride) {
  extern __shared__ __align__(16) unsigned char head_smem[];
  const int HP = H + kHeadPad;
  uint16_t* hs = reinterpret_cast<uint16_t*>(head_smem);
  SoftStat* red = reinterpret_cast<SoftStat*>(head_smem + sizeof(uint16_t) * kHeadTokChunk * HP);

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;

  const long NC = (V + 16 * QG - 1) / (16 * QG);
  const long NW = static_cast<long>(gridDim.x) * kHeadWaves;
  const long wid = static_cast<long>(blockIdx.x) * kHeadWaves + wave;
  const int c0 = static_cast<int>(wid * NC / NW);
  const int c1 = static_cast<int>((wid + 1) * NC / NW);
  const int KS = H / 32;
  const int nb = KS / U;                        // k-batches per chunk (even iff NBEVEN)
  const int iters = (c1 - c0) * nb;

  // fragment pointer of chunk ch, group q (row-major: a row past V reads
  // row V-1; packed: a group past the last one reads the last one; both are
  // dropped in the epilogue, which keeps only v < V)
  const long ngroups = (V + 15) / 16;            // 16-row groups (packed: padded rows)
  auto wfrag = [&](int ch, int q) {
    long grp = static_cast<long>(ch) * QG + q;
    if (layout == BDM_LAYOUT_MFMA_TILES) {
      grp = grp < ngroups ? grp : ngroups - 1;   // chunk past the last group: dropped later
      return frag_ptr(w, grp * 16, H, lane, layout);
    }
    const long v0 = grp * 16;
    long v = v0 + c;
    v = v < V ? v : V - 1;
    return FragPtr{w + v * H + g * 8, 32};
  };
  auto load_batch = [&](int it, u32x4(&b)[U][QG]) {
    const int ch = c0 + it / nb;
    const int s0 = (it % nb) * U;
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const FragPtr f = wfrag(ch, q);
#pragma unroll
      for (int u = 0; u < U; ++u) b[u][q] = ld16_stream(f.p + (s0 + u) * f.step);
    }
  };

  // the first two batches in flight before the staging barrier
  u32x4 bcur[U][QG], bnxt[U][QG];
  if (iters > 0) load_batch(0, bcur);
  if (iters > 1) load_batch(1, bnxt);

  // stage this pass's hidden rows (rows >= ntok are zero): every load first
  // (clamped addresses, no branches), then the LDS stores
  {
    constexpr int kStage = kHeadTokChunk * BDM_MAX_HIDDEN / 8 / (kHeadWaves * 64);
    const int c8n = H / 8;
    const int total = kHeadTokChunk * c8n;
    u32x4 v[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = tid + j * kHeadWaves * 64;
      const int r = idx / c8n;
      const int c8 = idx - r * c8n;
      const bool ok = idx < total && r < ntok;
      const u32x4 x = ld16(h + static_cast<size_t>(tok0 + (ok ? r : 0)) * H + (ok ? c8 : 0) * 8);
      v[j] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = tid + j * kHeadWaves * 64;
      if (idx < total) {
        const int r = idx / c8n;
        *reinterpret_cast<u32x4*>(hs + r * HP + (idx - r * c8n) * 8) = v[j];
      }
    }
  }
  __syncthreads();

  const uint16_t* arow0 = hs + c * HP + g * 8;
  const uint16_t* arow1 = hs + (16 + c) * HP + g * 8;

  SoftStat st[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) st[mt][i] = softstat_empty();

  f32x4 acc[QG][2];
#pragma unroll
  for (int q = 0; q < QG; ++q)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int it, const u32x4(&b)[U][QG]) {
    const int s0 = (it % nb) * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(arow0 + (s0 + u) * 32);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(arow1 + (s0 + u) * 32);
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        acc[q][0] = mfma_bf16(a0, b[u][q], acc[q][0]);
        acc[q][1] = mfma_bf16(a1, b[u][q], acc[q][1]);
      }
    }
  };
  // after the last k-batch of a chunk: fold its logits into the online
  // softmax state (branch-free; columns past V and the mask column count as
  // -inf).  Per lane the vocabulary id only grows, so the strict '>' keeps
  // the lowest id among equal maxima.
  auto finish = [&](int it) {
    if (it % nb != nb - 1) return;
    const int ch = c0 + it / nb;
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int v = (ch * QG + q) * 16 + c;
      const bool valid = v < V && v + voff != mask_id;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          SoftStat& st_ = st[mt][i];
          const float l = valid ? acc[q][mt][i] : -INFINITY;
          const float nm = fmaxf(st_.m, l);
          const float sc = (st_.m == nm) ? 1.0f : expf(st_.m - nm);
          const float add = (l == -INFINITY) ? 0.0f : expf(l - nm);
          st_.a = (l > st_.m) ? v + voff : st_.a;
          st_.s = st_.s * sc + add;
          st_.m = nm;
        }
        acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  // ping-pong batches: while one is multiplied the other is loading.  With
  // an even number of k-batches per chunk a chunk never ends on an even
  // iteration, so those steps carry no epilogue.
  if (iters == 1) {
    compute(0, bcur);
    finish(0);
  } else if (iters > 1) {
    int it = 0;
    for (; it + 3 < iters; it += 2) {
      compute(it, bcur);
      load_batch(it + 2, bcur);
      if (!NBEVEN) finish(it);
      compute(it + 1, bnxt);
      load_batch(it + 3, bnxt);
      finish(it + 1);
    }
    compute(it, bcur);
    if (it + 2 < iters) {
      load_batch(it + 2, bcur);
      finish(it);
      compute(it + 1, bnxt);
      finish(it + 1);
      compute(it + 2, bcur);
      finish(it + 2);
    } else {
      finish(it);
      compute(it + 1, bnxt);
      finish(it + 1);
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
    const size_t o = static_cast<size_t>(tok0 + tid) * pstride + chk(blockIdx.x, pstride, kChkStat);
    pm[o] = s.m;
    ps[o] = s.s;
    pa[o] = s.a;
  }
}

// Cooperative variant for H % 256 == 0 (KSW = H / 256 k-steps per wave):
// the 8 waves of a workgroup stream every 16-row group together, wave w the
// k-steps [w*KSW, (w+1)*KSW), with that slice of the hidden rows (MT tiles
// of 16 rows: 32 or 64 rows per pass over the weights) held in its
// registers for the whole run.  The 8 partial products of a group meet in
// LDS and are summed in wave order, and each (token, column) of the group is
// folded into the online-softmax state of one lane (for f < MT/2: token
// 16 (2f + w/4) + 4 (lane/16) + w%4, column lane%16, so the 64 lanes of a
// wave read 64 consecutive partials).  The workgroup takes one contiguous
// run of groups; its waves move in step (one barrier per group), and the
// loads of the next two groups are in flight while a group is reduced.
// Loads past the run read the hidden rows instead (valid, L2-resident,
// ignored), so no load sits behind a branch.
//
// VERIFY (the verify epilogue): no row is masked and the state is a VStat
// (adds q = sum e^(l-m)(l-m) and the logit of the row's candidate cand[t]).
//
// Several passes in one launch (npass > 1, rows [tok0, tok0 + ntok) cut into
// npass passes of rpp rows): the vocabulary keeps its gridDim.x ranges, and
// the npass workgroups that run the passes of a group of npass consecutive
// ranges sit on one XCD (workgroup b runs on XCD b % 8) and start together,
// so the weights they stream are read from HBM about once and from L2 by the
// others (REUSE: loads that allocate in the caches).  Each workgroup streams
// its ranges back to back and writes one partial per (row, range), the same
// numbers as one launch per pass.
template <int KSW, int MT, bool VERIFY, bool REUSE>
__global__ __launch_bounds__(kHeadWaves * 64, 1) void head_coop_kernel(
    const uint16_t* __restrict__ h, int H, const uint16_t* __restrict__ w, int V, int voff,
    int layout, int32_t mask_id, int tok0, int ntok, int npass, int rpp,
    float* __restrict__ pm, float* __restrict__ ps, int32_t* __restrict__ pa, int pstride,
    const int32_t* __restrict__ cand, int ncand, float* __restrict__ pq,
    float* __restrict__ plc) {
  static_assert(kHeadWaves == 8 && (MT == 2 || MT == 4), "4 token rows of a tile per wave");
  constexpr int NF = MT / 2;                                   // tokens folded per lane
  __shared__ float part[2][kHeadWaves][MT][4][kWave];          // 16 KB per tile

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  // this workgroup's pass and first range (one pass per launch unless REUSE)
  const int np = REUSE ? npass : 1;
  int pass = 0, qa = blockIdx.x;
  if (np > 1) {
    const int i = static_cast<int>(blockIdx.x) / 8;
    const int per_xcd = static_cast<int>(gridDim.x) / 8 / np;   // range groups per XCD
    pass = i % np;
    qa = (static_cast<int>(blockIdx.x % 8) * per_xcd + i / np) * np;
  }
  const int pt0 = tok0 + pass * rpp;                            // this pass's rows
  const int rem = tok0 + ntok - pt0;
  const int pn = np == 1 ? ntok : (rem < rpp ? rem : rpp);
  if (pn <= 0) return;
  const long ngroups = (V + 15) / 16;
  auto bound = [&](int q) -> long { return static_cast<long>(q) * ngroups / gridDim.x; };
  const long G0 = bound(qa);
  const long G1 = bound(qa + np);
  const int n = static_cast<int>(G1 - G0);
  const int s0 = wave * KSW;

  // weight fragments of group gi (n <= gi: the hidden rows, never used)
  auto wfrag = [&](long gi) -> FragPtr {
    if (gi >= G1) return FragPtr{h + c * 8, 0};
    gi = chk(gi, ngroups, kChkVocabRow);
    if (layout == BDM_LAYOUT_MFMA_TILES) return frag_ptr(w, gi * 16, H, lane, layout);
    long v = gi * 16 + c;
    v = v < V ? v : V - 1;
    return FragPtr{w + v * H + g * 8, 32};
  };
  auto load = [&](long gi, u32x4(&b)[KSW]) {
    const FragPtr f = wfrag(gi);
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
      if constexpr (REUSE) b[s] = ld16(f.p + (s0 + s) * f.step);
      else b[s] = ld16_stream(f.p + (s0 + s) * f.step);
    }
  };
  // NB groups of weights in flight (ping-pong, or three buffers when the
  // 32-row tile leaves the registers for it)
#ifndef BDM_HEAD_BUFS
#define BDM_HEAD_BUFS 2
#endif
  constexpr int NB = MT == 2 ? BDM_HEAD_BUFS : 2;
  u32x4 bufs[NB][KSW];
#pragma unroll
  for (int u = 0; u < NB; ++u) load(G0 + u, bufs[u]);
  // this wave's slice of the hidden rows (rows >= ntok are zero)
  u32x4 a[MT][KSW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bool ok = 16 * mt + c < pn;
    const uint16_t* r = h + static_cast<size_t>(pt0 + (ok ? 16 * mt + c : 0)) * H + g * 8;
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
      const u32x4 x = ld16(r + (s0 + s) * 32);
      a[mt][s] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // the (token, column) pairs this lane folds: tokens ot[f], column c
  SoftStat st[NF];
  VStat vs[NF];
  int mycand[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ot = 16 * (2 * f + (wave >> 2)) + 4 * g + (wave & 3);
    st[f] = softstat_empty();
    vs[f] = vstat_empty();
    mycand[f] = -1;
    if (VERIFY) mycand[f] = (pt0 + ot < ncand && ot < pn) ? cand[pt0 + ot] : -1;
  }

  // fold group j's partial products (in LDS buffer j & 1) into the lanes'
  // online-softmax states
  auto fold = [&](int j) {
    const int v = static_cast<int>((G0 + j) * 16) + c;
    const bool live = v < V && v + voff != mask_id;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int ot = 16 * (2 * f + (wave >> 2)) + 4 * g + (wave & 3);
      const int omt = ot >> 4, oq = (ot >> 2) & 3, oi = ot & 3;
      float l = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kHeadWaves; ++wv) l += part[j & 1][wv][omt][oi][16 * oq + c];
      if (!live) l = -INFINITY;
      if constexpr (VERIFY) {
        // q += exp(l - m)(l - m) under the same rescaling as s
        VStat& x = vs[f];
        const float nm = fmaxf(x.m, l);
        if (nm != -INFINITY) {
          const float d = x.m - nm;                     // <= 0; -inf while empty
          const float sc = (x.m == -INFINITY) ? 0.0f : expf(d);
          const float add = (l == -INFINITY) ? 0.0f : expf(l - nm);
          x.q = (x.m == -INFINITY ? 0.0f : sc * (x.q + d * x.s)) +
                (l == -INFINITY ? 0.0f : add * (l - nm));
          x.s = x.s * sc + add;
          x.a = (l > x.m) ? v + voff : x.a;
          x.m = nm;
        }
        if (v + voff == mycand[f]) x.lc = l;
      } else {
        SoftStat& x = st[f];
        const float nm = fmaxf(x.m, l);
        const float sc = (x.m == nm) ? 1.0f : expf(x.m - nm);
        const float add = (l == -INFINITY) ? 0.0f : expf(l - nm);
        x.a = (l > x.m) ? v + voff : x.a;
        x.s = x.s * sc + add;
        x.m = nm;
      }
    }
  };
  // the group's products (and the next loads), into LDS buffer j & 1
  auto mma = [&](int j, u32x4(&b)[KSW], f32x4(&acc)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSW; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(a[mt][s], b[s], acc[mt]);
    load(G0 + j + NB, b);
  };
  auto store = [&](int j, const f32x4(&acc)[MT]) {
    float* pp = &part[j & 1][wave][0][0][0];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[(mt * 4 + i) * kWave + lane] = acc[mt][i];
  };
  auto step = [&](int j, u32x4(&b)[KSW]) {
    f32x4 acc[MT];
    mma(j, b, acc);
    store(j, acc);
    __syncthreads();
    fold(j);
  };
  // the partials of range q for this lane's tokens (the 16 columns of a
  // token sit in one DPP row, each token in one wave)
  auto write_partials = [&](int q) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int ot = 16 * (2 * f + (wave >> 2)) + 4 * g + (wave & 3);
      const size_t o = static_cast<size_t>(pt0 + ot) * pstride + chk(q, pstride, kChkStat);
      if constexpr (VERIFY) {
        const VStat r = row_merge_vstat(vs[f]);
        if (c == 0 && ot < pn) {
          pm[o] = r.m;
          ps[o] = r.s;
          pa[o] = r.a;
          pq[o] = r.q;
          plc[o] = r.lc;
        }
      } else {
        const SoftStat r = row_merge_stat(st[f]);
        if (c == 0 && ot < pn) {
          pm[o] = r.m;
          ps[o] = r.s;
          pa[o] = r.a;
        }
      }
    }
  };
  if constexpr (!REUSE) {
    int j = 0;
    for (; j + NB - 1 < n; j += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) step(j + u, bufs[u]);
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (j + u < n) step(j + u, bufs[u]);
    write_partials(blockIdx.x);
  } else {
    // range qa + qi ends before group nb (relative to G0); flush writes its
    // partials and starts the next range
    int qi = 0;
    long nb = bound(qa + 1) - G0;
    auto flush = [&]() {
      write_partials(qa + qi);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        st[f] = softstat_empty();
        vs[f] = vstat_empty();
      }
      ++qi;
      nb = bound(qa + qi + 1) - G0;
    };
    // ranges that end at or before group jj (workgroup-uniform)
    auto advance = [&](int jj) {
      while (qi < np - 1 && jj >= nb) flush();
    };
    // software-pipelined: group j's products are computed while group j-1
    // is folded (its partials were published by the previous barrier), so
    // the fold's LDS reads and exponentials hide behind the MFMAs
    auto pstep = [&](int j, u32x4(&b)[KSW]) {
      f32x4 acc[MT];
      mma(j, b, acc);
      if (j > 0) fold(j - 1);
      store(j, acc);
      advance(j);                      // ranges that end with group j - 1
      __syncthreads();
    };
    int j = 0;
    for (; j + NB - 1 < n; j += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) pstep(j + u, bufs[u]);
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (j + u < n) pstep(j + u, bufs[u]);
    if (n > 0) fold(n - 1);
    while (qi < np) flush();
  }
}

// One workgroup.  16 threads (one DPP row) per token merge that token's
// partials (all loads issued first), the row reduction finishes the merge,
// and the commit rule is applied to every block of B rows on its own (B >= T:
// the whole call is one block), a wave per block.
__global__ __launch_bounds__(1024) void head_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const int32_t* __restrict__ pa,
    int T, int nparts, int pstride, int32_t mask_id, float threshold, int fallback, int B,
    int32_t* tokens,
    int32_t* __restrict__ argmax_out, float* __restrict__ conf_out,
    int32_t* __restrict__ n_committed, int32_t* __restrict__ n_left) {
  extern __shared__ float smem[];
  float* sconf = smem;                                   // [T]
  int* sarg = reinterpret_cast<int*>(smem + T);         // [T]
  int* stok = sarg + T;                                  // [T]
  const int tid = threadIdx.x;
  for (int t = tid; t < T; t += blockDim.x) stok[t] = tokens[t];

  const int sub = tid & 15;          // thread within the token's row
  for (int t0 = 0; t0 < T; t0 += blockDim.x >> 4) {
    const int t = t0 + (tid >> 4);
    // a wave holds 4 rows; a wave with none skips the merge (the merge is
    // VALU-bound on this one CU)
    if (t0 + (tid / kWave) * (kWave / 16) >= T) continue;
    const bool on = t < T;           // row-uniform
    const size_t base = static_cast<size_t>(on ? t : 0) * pstride;
    SoftStat st = softstat_empty();
    for (int i0 = 0; i0 < nparts; i0 += 16 * 16) {
      SoftStat part[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 16 + sub;
        const size_t ix = base + chk(i < nparts ? i : 0, pstride, kChkStat);
        part[u] = (on && i < nparts) ? SoftStat{pm[ix], ps[ix], pa[ix]} : softstat_empty();
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) st = softstat_merge(st, part[u]);
    }
    st = row_merge_stat(st);
    if (on && sub == 0) {
      // a row with a finite maximum has s >= 1 (its maximum contributes
      // e^0); no finite logit (s = 0, id INT32_MAX) or a NaN sum gives no
      // prediction: argmax -1, conf 0, and the rule never commits it
      const bool ok = st.a != INT32_MAX && st.s >= 1.0f;
      const float cf = ok ? 1.0f / st.s : 0.0f;
      const int a = ok ? st.a : -1;
      sconf[t] = cf;
      sarg[t] = a;
      if (argmax_out) argmax_out[t] = a;
      if (conf_out) conf_out[t] = cf;
    }
  }
  __syncthreads();

  // Commit rule per block of B rows, wave w taking blocks w, w + 16, ...
  // Best masked row of a block for the fallback: largest conf, equal ->
  // lowest position.
  __shared__ int wsum[2][1024 / kWave];
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int nw = static_cast<int>(blockDim.x) / kWave;
  const int nblk = (T + B - 1) / B;
  int wcommit = 0, wleft = 0;
  for (int b = wave; b < nblk; b += nw) {
    const int r0 = b * B;
    const int r1 = (T - r0) < B ? T : r0 + B;
    int ncommit = 0, nmasked = 0;
    float best_c = -INFINITY;
    int best_t = INT32_MAX;
    for (int t0 = r0; t0 < r1; t0 += kWave) {
      const int t = t0 + lane;
      const bool m = t < r1 && stok[t] == mask_id;
      int commit = 0;
      nmasked += wave_sum_i(m ? 1 : 0);
      if (m && sarg[t] >= 0) {
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
      if (lane == 0) {
        const int bt = chk(best_t, T, kChkTokenRow);
        tokens[bt] = sarg[bt];
      }
      ncommit = 1;
    }
    wcommit += ncommit;
    wleft += nmasked - ncommit;
  }
  if (lane == 0) {
    wsum[0][wave] = wcommit;
    wsum[1][wave] = wleft;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0, l = 0;
    for (int w = 0; w < nw; ++w) {
      c += wsum[0][w];
      l += wsum[1][w];
    }
    if (n_committed) *n_committed = c;
    if (n_left) *n_left = l;
  }
}

// Verify epilogue ([files] "Two ways to run it"), one workgroup: merge the
// statistics of each of the T1 rows (16 threads per row, fixed tree), then
// accept_t (t < T1 - 1) by the rule, r = the accepted prefix, and the
// round's tokens: candidates 0..r-1, the most likely token of row r, -1 after.
//   rule 0 (exact):     cand_t == argmax_t
//   rule 1 (threshold): p_t(cand_t) >= min(ratio, delta * exp(-H_t)),
//                       p = exp(lc - m) / s, H = log s - q / s
__global__ __launch_bounds__(1024) void verify_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const int32_t* __restrict__ pa,
    const float* __restrict__ pq, const float* __restrict__ plc, int T1, int nparts, int pstride,
    const int32_t* __restrict__ cand, int V, int rule, float ratio, float delta,
    int32_t* __restrict__ tokens_out, int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ accept_out, int32_t* __restrict__ argmax_out,
    float* __restrict__ pcand_out, float* __restrict__ entropy_out) {
  extern __shared__ int vsm[];
  int* sacc = vsm;                 // [T1]
  int* sarg = vsm + T1;            // [T1]
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  for (int t0 = 0; t0 < T1; t0 += blockDim.x >> 4) {
    const int t = t0 + (tid >> 4);
    if (t0 + (tid / kWave) * (kWave / 16) >= T1) continue;   // a wave with no row
    const bool on = t < T1;          // row-uniform
    const size_t base = static_cast<size_t>(on ? t : 0) * pstride;
    VStat st = vstat_empty();
    for (int i0 = 0; i0 < nparts; i0 += 16 * 8) {
      VStat part[8];                 // all loads of a batch issued before merging
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 16 + sub;
        part[u] = (on && i < nparts) ? VStat{pm[base + i], ps[base + i], pq[base + i],
                                             pa[base + i], plc[base + i]}
                                     : vstat_empty();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) st = vstat_merge(st, part[u]);
    }
    st = row_merge_vstat(st);
    if (on && sub == 0) {
      // no finite logit, or a NaN sum: no prediction (argmax -1), rejected
      const bool ok = st.a != INT32_MAX && st.s >= 1.0f;
      const int am = ok ? st.a : -1;
      const float ent = logf(st.s) - st.q / st.s;
      const float pc = expf(st.lc - st.m) / st.s;
      int acc = 0;
      if (t < T1 - 1) {
        const int c = cand[t];
        acc = (!ok || c < 0 || c >= V) ? 0
              : (rule == 0)            ? (c == am ? 1 : 0)
                                       : (pc >= fminf(ratio, delta * expf(-ent)) ? 1 : 0);
        if (accept_out) accept_out[t] = acc;
        if (pcand_out) pcand_out[t] = pc;
      }
      sacc[t] = acc;
      sarg[t] = am;
      if (argmax_out) argmax_out[t] = am;
      if (entropy_out) entropy_out[t] = ent;
    }
  }
  __syncthreads();
  if (tid >= kWave) return;
  // the accepted prefix: the first rejected row (row T1-1 never accepts)
  const int lane = tid;
  int first = T1 - 1;
  for (int t0 = 0; t0 < T1; t0 += kWave) {
    const int t = t0 + lane;
    const unsigned long long rej = __ballot(t < T1 && !sacc[t]);
    if (rej) {
      first = t0 + __builtin_ctzll(rej);
      break;
    }
  }
  for (int t = lane; t < T1; t += kWave)
    tokens_out[t] = t < first ? cand[t] : (t == first ? sarg[t] : -1);
  if (lane == 0) *n_accepted = first;
}

void launch_verify_merge(const float* pm, const float* ps, const int32_t* pa, const float* pq,
                         const float* plc, int T1, int parts, int pstride, const int32_t* cand,
                         int V, int rule, float ratio, float delta, int32_t* tokens_out,
                         int32_t* n_accepted, int32_t* accept_out, int32_t* argmax_out,
                         float* pcand_out, float* entropy_out, hipStream_t s) {
  verify_merge_kernel<<<1, 1024, static_cast<size_t>(T1) * 8, s>>>(
      pm, ps, pa, pq, plc, T1, parts, pstride, cand, V, rule, ratio, delta, tokens_out, n_accepted,
      accept_out, argmax_out, pcand_out, entropy_out);
}

// the k-batch must divide H/32 (always even), else batches of 2 k-steps
using HeadKernel = void (*)(const uint16_t*, int, const uint16_t*, int, int, int, int32_t, int, int,
                            float*, float*, int32_t*, int);
static const HeadKernel kHeadKernels[4] = {
    &head_tile_kernel<kHeadQG, kHeadU, true>, &head_tile_kernel<kHeadQG, kHeadU, false>,
    &head_tile_kernel<kHeadQG, 2, true>, &head_tile_kernel<kHeadQG, 2, false>};

static HeadKernel head_kernel_for(int H) {
  const int KS = H / 32;
  const int u = (KS % kHeadU == 0) ? kHeadU : 2;
  const bool even = (KS / u) % 2 == 0;
  return kHeadKernels[(u == kHeadU ? 0 : 2) + (even ? 0 : 1)];
}

// ---- many rows: the head as a tiled GEMM ----------------------------------
// From kGmMinRows rows (several blocks in one call) the head has enough rows
// to be bound by the MFMA units and the caches, not by HBM: 2 * rows * V * H
// flops over a gigabyte of weights.  Workgroup (range q, row block mb): the
// 256 rows of block mb against the vocabulary range q (the same 16-row
// groups as the persistent kernel's workgroup q, so the partials have the
// same meaning), in chunks of 256 vocabulary rows, each chunk over the whole
// K = H.  A stage is one MFMA k-step: 16 tiles of hidden rows and 16 of
// vocabulary rows (16 x 32 each, 1 KB), loaded straight into LDS in MFMA
// operand order (global_load_lds: lane l's 16 bytes land at l * 16, so the
// operand reads are conflict-free 16-byte reads); four stage buffers, the
// loads of the next three stages in flight while one is multiplied, one
// barrier per stage.  Wave (wm, wn) of the 8 owns rows 64 wm .. +63 and
// vocabulary rows 128 wn .. +127 of the chunk: 4 x 8 accumulator tiles, 12
// KB of LDS reads for 32 MFMAs per k-step.  The chunk's logits never leave
// the accumulators: each lane folds its 8 logits per row into its own
// online-softmax state of that row (max, sum of exp, argmax; the mask token
// and rows past the range at -inf, NaN as -inf), and after the last chunk the
// 16 lanes of a row and the two vocabulary halves are merged in a fixed tree.
// The row blocks of one range run next to each other on one XCD (workgroup b
// on XCD b % 8), so a chunk's weights come from HBM about once and from L2
// for the other row blocks.
constexpr int kGmBM = 256;          // hidden rows per workgroup
constexpr int kGmBN = 256;          // vocabulary rows per chunk
constexpr int kGmBK = 32;           // k per stage (one MFMA k-step)
constexpr int kGmTiles = 32;        // 1 KB operand tiles per stage: 16 of rows, 16 of vocabulary
#ifndef BDM_HEAD_GEMM_BUFS
#define BDM_HEAD_GEMM_BUFS 4
#endif
constexpr int kGmBufs = BDM_HEAD_GEMM_BUFS;   // stage buffers: all but one in flight (4 or 5)
static_assert(kGmBufs == 4 || kGmBufs == 5, "four or five stage buffers");
#ifndef BDM_HEAD_GEMM_MIN_T
#define BDM_HEAD_GEMM_MIN_T 256
#endif
constexpr int kGmMinRows = BDM_HEAD_GEMM_MIN_T;
#ifndef BDM_HEAD_GEMM_MGROUP
#define BDM_HEAD_GEMM_MGROUP 0      // row blocks per group (0: all of them)
#endif

// fold the 8 logits of one row this lane holds (vocabulary ids v0 + 16 j,
// increasing) into this lane's running state of the row (max, sum of exp
// relative to it, argmax; ids increase from chunk to chunk, so a strictly
// larger value is what moves the argmax and equal maxima keep the lowest id)
__device__ __forceinline__ void gm_fold_lane(const float (&l)[8], long v0, long vend, int voff,
                                             int32_t mask_id, float& m, float& s, int& a) {
  constexpr float kLog2e = 1.4426950408889634f;
  float x[8];
  float cm = -INFINITY;
  int ca = INT32_MAX;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const long v = v0 + 16 * j;
    const bool live = v < vend && static_cast<long>(voff) + v != mask_id && l[j] == l[j];
    x[j] = live ? l[j] : -INFINITY;
    if (x[j] > cm) {
      cm = x[j];
      ca = static_cast<int>(v) + voff;
    }
  }
  if (cm > m) {                                    // a new maximum: rescale the sum
    s = (m == -INFINITY) ? 0.0f : s * exp2f((m - cm) * kLog2e);
    m = cm;
    a = ca;
  }
  if (m != -INFINITY) {
    const float m2 = m * kLog2e;
    float add = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) add += (x[j] == -INFINITY) ? 0.0f : exp2f(fmaf(x[j], kLog2e, -m2));
    s += add;
  }
}

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// A workgroup barrier that orders memory operations in the compiler but
// waits for nothing itself: the stage loads that must have landed are
// waited for explicitly before it (__syncthreads would wait for every load
// into LDS still in flight, the stages ahead included).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

__global__ __launch_bounds__(512, 2) void head_gemm_kernel(
    const uint16_t* __restrict__ h, int T, int H, const uint16_t* __restrict__ w, int V,
    int voff, int layout, int32_t mask_id, int tok0, int P, float* __restrict__ pm,
    float* __restrict__ ps, int32_t* __restrict__ pa, int pstride) {
  // the stage buffers as separate arrays: the loads into all but one of
  // them are in flight while that one is read
  __shared__ u32x4 lds0[kGmTiles][kWave];                       // 32 KB each
  __shared__ u32x4 lds1[kGmTiles][kWave];
  __shared__ u32x4 lds2[kGmTiles][kWave];
  __shared__ u32x4 lds3[kGmTiles][kWave];
  __shared__ u32x4 lds4[kGmBufs == 5 ? kGmTiles : 1][kWave];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int wm = wave & 3;
  const int wn = wave >> 2;
  const int nmb = (T + kGmBM - 1) / kGmBM;
  // XCD x (workgroup b runs on XCD b % 8) takes ranges [x P/8, (x+1) P/8);
  // its workgroups run the ranges for a group of G row blocks at a time,
  // the G row blocks of one range consecutive (they share the range's
  // weights through L2; fewer row blocks at a time keep their hidden rows
  // in L2)
  int q, mb;
  if (P % 8 == 0) {
    const int x = static_cast<int>(blockIdx.x % 8), i = static_cast<int>(blockIdx.x / 8);
    const int R8 = P / 8;
    int G = BDM_HEAD_GEMM_MGROUP;
    G = (G <= 0 || G > nmb) ? nmb : G;
    const int per = R8 * G;                                     // items of a full group
    const int mg = i / per, rem = i % per;
    const int gsz = (mg * G + G <= nmb) ? G : nmb - mg * G;     // the last group may be short
    q = x * R8 + rem / gsz;
    mb = mg * G + rem % gsz;
  } else {
    q = static_cast<int>(blockIdx.x) / nmb;
    mb = static_cast<int>(blockIdx.x) % nmb;
  }
  if (q >= P) return;                                            // (grid = nmb * P)
  const long ngroups = (V + 15) / 16;
  const long G0 = static_cast<long>(q) * ngroups / P;
  const long G1 = static_cast<long>(q + 1) * ngroups / P;
  const long vend = G1 * 16 < V ? G1 * 16 : V;                   // this range: [16 G0, vend)
  const int nchunk = static_cast<int>((G1 - G0 + 15) / 16);
  const int rb = mb * kGmBM;                                      // first row of the block
  const int KST = H / kGmBK;                                      // stages per chunk
  const int total = nchunk * KST;

  // loads of a stage: waves 0-3 the 16 hidden-row tiles (wave w: row tiles
  // 4w .. 4w+3), waves 4-7 the 16 vocabulary tiles; lane l's 16 bytes land
  // at l * 16 of the tile (the MFMA operand order)
  const bool rows_side = wave < 4;
  const int t16 = (wave & 3) * 4;                                 // first 16-row tile
  const bool packed = !rows_side && layout == BDM_LAYOUT_MFMA_TILES;
  const int sstride = packed ? 512 : kGmBK;                       // elements per stage
  const uint16_t* base[4];                                        // k = 0 of tile row u
  if (rows_side) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int r = rb + (t16 + u) * 16 + c;
      r = r < T ? r : T - 1;
      base[u] = h + static_cast<size_t>(tok0 + r) * H + g * 8;
    }
  }
  auto chunk_rows = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      long gi = G0 + ch * 16 + t16 + u;
      gi = chk(gi < ngroups ? gi : ngroups - 1, ngroups, kChkVocabRow);
      if (packed) {
        base[u] = w + static_cast<size_t>(gi) * (H / 32) * 512 + lane * 8;
      } else {
        long v = gi * 16 + c;
        v = v < V ? v : V - 1;
        base[u] = w + static_cast<size_t>(v) * H + g * 8;
      }
    }
  };
  const int tbase = (rows_side ? 0 : 16) + t16;
  auto stage = [&](int it, u32x4 (*buf)[kWave]) __attribute__((always_inline)) {
    const int st = it % KST;
    if (st == 0 && !rows_side) chunk_rows(it / KST);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(base[u] + st * sstride),
          (__attribute__((address_space(3))) void*)&buf[tbase + u][0], 16, 0, 0);
  };

  // this lane's running state of its 16 rows (row tile i, row 4 g + e)
  float sm[16], ss[16];
  int sa[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sm[r] = -INFINITY;
    ss[r] = 0.0f;
    sa[r] = INT32_MAX;
  }
  f32x4 acc[4][8];
  auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto mma = [&](u32x4 (*buf)[kWave]) __attribute__((always_inline)) {
    u32x4 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = buf[wm * 4 + i][lane];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 b = buf[16 + wn * 8 + j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_bf16(a[i], b, acc[i][j]);
    }
  };
  auto fold = [&](int ch) __attribute__((always_inline)) {
    const long v0 = (G0 + ch * 16) * 16 + wn * 128 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float l[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) l[j] = acc[i][j][e];
        gm_fold_lane(l, v0, vend, voff, mask_id, sm[i * 4 + e], ss[i * 4 + e], sa[i * 4 + e]);
      }
  };
  // stage it: stage it + NB - 1's loads first, then this one's products (a
  // finished chunk folded); then this wave's loads of stage it + 1 are
  // waited for (those of the later stages stay in flight) and the barrier
  // makes every wave's visible
  // (every step issues four loads, branch-free, so that the compiler can
  // count them: past the last stage it loads the last one again into the
  // buffer no stage uses any more)
  constexpr int NB = kGmBufs;
  auto step = [&](int it, u32x4 (*cur)[kWave], u32x4 (*ahead)[kWave]) __attribute__((always_inline)) {
    stage(it + NB - 1 < total ? it + NB - 1 : total - 1, ahead);
    mma(cur);
    if ((it + 1) % KST == 0) {
      fold(it / KST);
      zero();
    }
    wait_vmcnt<4 * (NB - 2)>();
    stage_barrier();
  };
  auto last = [&](int it) { return it < total ? it : total - 1; };

  if (total > 0) {
    stage(0, lds0);
    stage(last(1), lds1);
    stage(last(2), lds2);
    if constexpr (NB == 5) stage(last(3), lds3);
    wait_vmcnt<4 * (NB - 2)>();
    stage_barrier();
    zero();
    int it = 0;
    if constexpr (NB == 4) {
      for (; it + 3 < total; it += 4) {
        step(it, lds0, lds3);
        step(it + 1, lds1, lds0);
        step(it + 2, lds2, lds1);
        step(it + 3, lds3, lds2);
      }
      if (it < total) step(it, lds0, lds3);
      if (it + 1 < total) step(it + 1, lds1, lds0);
      if (it + 2 < total) step(it + 2, lds2, lds1);
    } else {
      for (; it + 4 < total; it += 5) {
        step(it, lds0, lds4);
        step(it + 1, lds1, lds0);
        step(it + 2, lds2, lds1);
        step(it + 3, lds3, lds2);
        step(it + 4, lds4, lds3);
      }
      if (it < total) step(it, lds0, lds4);
      if (it + 1 < total) step(it + 1, lds1, lds0);
      if (it + 2 < total) step(it + 2, lds2, lds1);
      if (it + 3 < total) step(it + 3, lds3, lds2);
    }
    wait_vmcnt<0>();                         // no load into LDS outlives the loop
  }
  // merge: the 16 lanes of each row (a fixed DPP tree), then the two
  // vocabulary halves
  SoftStat* red = reinterpret_cast<SoftStat*>(&lds0[0][0]);       // [2][kGmBM]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = i * 4 + e;
      const SoftStat x = row_merge_stat(SoftStat{sm[r], ss[r], sa[r]});
      if (c == 0) red[wn * kGmBM + wm * 64 + i * 16 + g * 4 + e] = x;
    }
  __syncthreads();
  if (tid < kGmBM && rb + tid < T) {
    const SoftStat x = softstat_merge(red[tid], red[kGmBM + tid]);
    const size_t o = static_cast<size_t>(tok0 + rb + tid) * pstride + chk(q, pstride, kChkStat);
    pm[o] = x.m;
    ps[o] = x.s;
    pa[o] = x.a;
  }
}

using CoopKernel = void (*)(const uint16_t*, int, const uint16_t*, int, int, int, int32_t, int,
                            int, int, int, float*, float*, int32_t*, int, const int32_t*, int,
                            float*, float*);

template <int MT, bool VERIFY, bool REUSE = false>
static CoopKernel coop_kernel_for(int H) {
  switch (H / 256) {
    case 1: return &head_coop_kernel<1, MT, VERIFY, REUSE>;
    case 2: return &head_coop_kernel<2, MT, VERIFY, REUSE>;
    case 4: return &head_coop_kernel<4, MT, VERIFY, REUSE>;
    case 8: return &head_coop_kernel<8, MT, VERIFY, REUSE>;
    default: return nullptr;
  }
}

constexpr int kCoopChunk = 64;   // rows per pass of the cooperative kernel (MT = 4)

void launch_head_stats(const uint16_t* h, int T, int H, const uint16_t* w, int V, int voff,
                       int layout, int32_t mask_id, float* pm, float* ps, int32_t* pa,
                       int pstride, int grid, hipStream_t s) {
#ifndef BDM_HEAD_COOP
#define BDM_HEAD_COOP 1
#endif
#ifndef BDM_HEAD_PASS_PAR
#define BDM_HEAD_PASS_PAR 1
#endif
  if (T >= kGmMinRows && H % kGmBK == 0 && grid >= 1 &&
      (layout == BDM_LAYOUT_ROW_MAJOR || layout == BDM_LAYOUT_MFMA_TILES)) {
    const int nmb = (T + kGmBM - 1) / kGmBM;
    head_gemm_kernel<<<nmb * grid, 512, 0, s>>>(h, T, H, w, V, voff, layout, mask_id, 0, grid,
                                                pm, ps, pa, pstride);
    return;
  }
  if (BDM_HEAD_COOP && H % 256 == 0 && coop_kernel_for<2, false>(H)) {
    // more rows than one pass takes: every pass in one launch (a power of
    // two of them, at most 32, so that whole groups of them fill each XCD)
    const int passes = (T + kCoopChunk - 1) / kCoopChunk;
    int np = 1;
    while (np < passes) np *= 2;
    if (BDM_HEAD_PASS_PAR && np > 1 && np <= 32 && grid % (8 * np) == 0) {
      const int rpp = (T + np - 1) / np;                  // <= kCoopChunk
      CoopKernel k = rpp <= 32 ? coop_kernel_for<2, false, true>(H)
                               : coop_kernel_for<4, false, true>(H);
      k<<<grid, kHeadWaves * 64, 0, s>>>(h, H, w, V, voff, layout, mask_id, 0, T, np, rpp, pm,
                                         ps, pa, pstride, nullptr, 0, nullptr, nullptr);
      return;
    }
    for (int t0 = 0; t0 < T; t0 += kCoopChunk) {
      const int n = (T - t0) < kCoopChunk ? (T - t0) : kCoopChunk;
      CoopKernel k = n <= 32 ? coop_kernel_for<2, false>(H) : coop_kernel_for<4, false>(H);
      k<<<grid, kHeadWaves * 64, 0, s>>>(h, H, w, V, voff, layout, mask_id, t0, n, 1, n, pm, ps,
                                         pa, pstride, nullptr, 0, nullptr, nullptr);
    }
    return;
  }
  HeadKernel tile = head_kernel_for(H);
  const size_t lds = head_lds_bytes(H);
  for (int t0 = 0; t0 < T; t0 += kHeadTokChunk) {
    const int n = (T - t0) < kHeadTokChunk ? (T - t0) : kHeadTokChunk;
    tile<<<grid, kHeadWaves * 64, lds, s>>>(h, H, w, V, voff, layout, mask_id, t0, n, pm, ps, pa,
                                            pstride);
  }
}

void launch_head_verify_stats(const uint16_t* h, int T, int H, const uint16_t* w, int V,
                              int layout, const int32_t* cand, int ncand, float* pm, float* ps,
                              int32_t* pa, float* pq, float* plc, int pstride, int grid,
                              hipStream_t s) {
  for (int t0 = 0; t0 < T; t0 += kCoopChunk) {
    const int n = (T - t0) < kCoopChunk ? (T - t0) : kCoopChunk;
    CoopKernel k = n <= 32 ? coop_kernel_for<2, true>(H) : coop_kernel_for<4, true>(H);
    k<<<grid, kHeadWaves * 64, 0, s>>>(h, H, w, V, 0, layout, -1, t0, n, 1, n, pm, ps, pa,
                                       pstride, cand, ncand, pq, plc);
  }
}

void launch_unmask(const float* pm, const float* ps, const int32_t* pa, int T, int parts,
                   int pstride, int32_t mask_id, float threshold, int fallback, int block,
                   int32_t* tokens, int32_t* argmax, float* conf, int32_t* n_committed,
                   int32_t* n_left, hipStream_t s) {
  const int B = (block <= 0 || block > T) ? T : block;
  head_merge_kernel<<<1, 1024, static_cast<size_t>(T) * 12, s>>>(
      pm, ps, pa, T, parts, pstride, mask_id, threshold, fallback, B, tokens, argmax, conf,
      n_committed, n_left);
}

int head_prepare() {
  const int lds = static_cast<int>(head_lds_bytes(BDM_MAX_HIDDEN));
  for (HeadKernel f : kHeadKernels)
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return -1;
  return 0;
}

BDM_DEBUG_WORD_READER(debug_words_head)

}  // namespace bdm
