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
// Work is indexed by the slot table of touched expert groups the select step
// builds ({expert, offset, count, slots of the group}; the shared expert,
// group E, first, then the heavy ones); workgroups past its end exit at once.  A workgroup loads
// its slot, the first token rows of its group, then its weight burst; no
// weight load sits behind a branch (k-steps past K read k-step 0 and are
// zeroed by a select), so the compiler keeps every load in flight.
// Activations and outputs are stored per
// (token, slot): row t*(k+1)+j for the j-th pick, t*(k+1)+k for the shared
// expert, so the combine reads each token's k+1 rows contiguously.
//
//   gateup_kernel   work item = (expert, 16 columns of I).  8 waves split
//                   K = H; each wave loads its whole K-slice of the 16 gate
//                   and 16 up rows in one burst, multiplies the expert's
//                   token tiles, and the partial sums meet in LDS where
//                   silu(g) * u is formed and stored as bf16.
//   down_kernel     work item = (expert, 32 rows of H).  Each wave owns 16
//                   output rows and the whole K = I; fp32 results per pair.
//   combine_kernel  y_t = bf16(r_t + sum_j w_tj Y_tj + Y_t,shared), fixed
//                   order, no atomics.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

constexpr int kGuCols = 16;     // I columns per gate/up work item
constexpr int kGuWaves = 8;     // waves splitting K in gate/up
constexpr int kGuMt = 2;        // 16-token tiles multiplied per pass
#ifndef BDM_DN_WAVES
#define BDM_DN_WAVES 2
#endif
constexpr int kDnWaves = BDM_DN_WAVES;  // waves per down work item, 16 rows of H each
constexpr int kDnRows = 16 * kDnWaves;  // H rows per down work item

// A slot names a real group: expert id in [0, E] (E only with a shared
// expert), 1 <= count, and its pair rows inside [0, P).
// (The end mark {-1, 0, 0, 0} is not a group; any other entry that fails
// is reported in the debug build.)
__device__ __forceinline__ bool slot_ok(int e, int off, int m, int E, int P, bool has_shared) {
  const bool ok =
      e >= 0 && (e < E || (e == E && has_shared)) && m >= 1 && off >= 0 && off <= P - m;
  if (!ok && !(e == -1 && off == 0 && m == 0)) note_oob(kChkSlot);
  return ok;
}

// A pair row read from the table, kept inside [0, P) (a row outside is
// reported in the debug build).
__device__ __forceinline__ int clamp_row(int r, int P) {
  if (r < 0 || r >= P) note_oob(kChkPairRow);
  return r < 0 ? 0 : (r >= P ? P - 1 : r);
}

// gate/up fragments.  In the pair layout the packed gate and up groups
// alternate in one buffer (w_up = w_gate + one group), so consecutive groups
// of either matrix are two groups apart.
__device__ __forceinline__ FragPtr frag_ptr_gu(const uint16_t* W, long row0, int K, int lane,
                                               int layout) {
  if (layout == BDM_LAYOUT_MFMA_TILES_GU)
    return {W + (row0 / 16) * 2 * (K / 32) * 512 + lane * 8, 512};
  return frag_ptr(W, row0, K, lane, layout);
}

// One k-step (8 consecutive k of one row) of a weight row.  With GUARD the
// k-step may lie past K: the load then reads k-step 0 (always valid) and the
// value is replaced by zeros, so no load sits behind a branch.
template <bool GUARD>
__device__ __forceinline__ u32x4 ld_kstep(FragPtr f, int s, int KS) {
  if (!GUARD) return ld16_stream(f.p + s * f.step);
  const bool on = s < KS;
  const u32x4 v = ld16_stream(f.p + (on ? s : 0) * f.step);
  return on ? v : u32x4{0u, 0u, 0u, 0u};
}

// work item = (touched group, 16 columns of I); KSW k-steps per wave
template <int KSW, bool GUARD>
__global__ __launch_bounds__(kGuWaves * 64, 4) void gateup_kernel(
    const uint16_t* __restrict__ x, int H, int I, int E, int k, int P, int layout,
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ ws_gate, const uint16_t* __restrict__ ws_up,
    const int4* __restrict__ slots, const int32_t* __restrict__ pair_rows,
    uint16_t* __restrict__ act) {
  __shared__ f32x4 red[kGuWaves][kGuMt][2][kWave];   // 32 KB
  __shared__ int srow[16 * kGuMt];

  const int tiles = I / kGuCols;
  const int4 slot = slots[blockIdx.x / tiles];
  const int e = slot.x;
  const int off = slot.y;
  const int m = slot.z;
  // past the touched groups (-1), or a slot that is not a valid group: every
  // index below stays inside its buffer whatever the table holds
  if (!slot_ok(e, off, m, E, P, ws_gate != nullptr)) return;
  const int n0 = (blockIdx.x % tiles) * kGuCols;
  const int K1 = k + 1;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int KS = H / 32;
  const int s0 = wave * KSW;

  // rows of the first token chunk before the weight burst (in-order
  // completion: waiting for them later does not wait for the weights)
  int row0 = clamp_row(pair_rows[off + (c < m ? c : 0)], P);
  int row1 = clamp_row(pair_rows[off + (16 + c < m ? 16 + c : 0)], P);

  const long wrow0 = (e == E) ? n0 : static_cast<long>(e) * I + n0;
  const FragPtr rg = frag_ptr_gu(e == E ? ws_gate : w_gate, wrow0, H, lane, layout);
  const FragPtr ru = frag_ptr_gu(e == E ? ws_up : w_up, wrow0, H, lane, layout);
  u32x4 bg[KSW], bu[KSW];
#pragma unroll
  for (int q = 0; q < KSW; ++q) {
    bg[q] = ld_kstep<GUARD>(rg, s0 + q, KS);
    bu[q] = ld_kstep<GUARD>(ru, s0 + q, KS);
  }

  for (int mc = 0; mc < m; mc += 16 * kGuMt) {
    if (mc > 0) {
      row0 = clamp_row(pair_rows[off + (mc + c < m ? mc + c : 0)], P);
      row1 = clamp_row(pair_rows[off + (mc + 16 + c < m ? mc + 16 + c : 0)], P);
    }
    if (wave == 0 && g == 0) {
      srow[c] = row0;
      srow[16 + c] = row1;
    }
    f32x4 ag0 = f32x4{0.f, 0.f, 0.f, 0.f}, au0 = ag0, ag1 = ag0, au1 = ag0;
#pragma unroll
    for (int mt = 0; mt < kGuMt; ++mt) {
      if (mt == 0 || mc + 16 < m) {               // workgroup-uniform
        const bool ok = mc + mt * 16 + c < m;
        const uint16_t* xr = x + static_cast<size_t>((mt == 0 ? row0 : row1) / K1) * H + g * 8;
        u32x4 a[KSW];
#pragma unroll
        for (int q = 0; q < KSW; ++q) {
          const int s = GUARD ? ((s0 + q) < KS ? s0 + q : 0) : s0 + q;
          const u32x4 v = ld16(xr + s * 32);
          a[q] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
        f32x4 accg = f32x4{0.f, 0.f, 0.f, 0.f}, accu = accg;
#pragma unroll
        for (int q = 0; q < KSW; ++q) {
          accg = mfma_bf16(a[q], bg[q], accg);
          accu = mfma_bf16(a[q], bu[q], accu);
        }
        if (mt == 0) {
          ag0 = accg;
          au0 = accu;
        } else {
          ag1 = accg;
          au1 = accu;
        }
      }
    }
    red[wave][0][0][lane] = ag0;
    red[wave][0][1][lane] = au0;
    red[wave][1][0][lane] = ag1;
    red[wave][1][1][lane] = au1;
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
        const int rl = mt * 16 + 4 * (ln >> 4) + q;
        if (mc + rl < m) {
          const float gv = gs[q];
          const float a = gv / (1.0f + expf(-gv)) * us[q];
          act[static_cast<size_t>(srow[rl]) * I + col] = f32_to_bf16(a);
        }
      }
    }
    __syncthreads();
  }
}

// work item = (touched group, kDnRows rows of H); each wave owns 16 output rows
// and the whole K = I (KS k-steps, KS <= KSMAX)
template <int KSMAX, bool GUARD>
__global__ __launch_bounds__(kDnWaves * 64, 2) void down_kernel(
    const uint16_t* __restrict__ act, int H, int I, int E, int P, int layout,
    const uint16_t* __restrict__ w_down, const uint16_t* __restrict__ ws_down,
    const int4* __restrict__ slots, const int32_t* __restrict__ pair_rows,
    float* __restrict__ ypair) {
  const int tiles = (H + kDnRows - 1) / kDnRows;
  const int4 slot = slots[blockIdx.x / tiles];
  const int e = slot.x;
  const int off = slot.y;
  const int m = slot.z;
  if (!slot_ok(e, off, m, E, P, ws_down != nullptr)) return;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int n0 = (blockIdx.x % tiles) * kDnRows + wave * 16;
  if (n0 >= H) return;                          // past H in the last tile (no barriers here)
  const int KS = I / 32;

  // rows of the first token tile (A operand row c; output rows 4g..4g+3)
  // before the weight burst
  int ra = clamp_row(pair_rows[off + (c < m ? c : 0)], P);
  int ro[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ro[q] = clamp_row(pair_rows[off + (4 * g + q < m ? 4 * g + q : 0)], P);

  const FragPtr rd = frag_ptr(e == E ? ws_down : w_down,
                             (e == E) ? n0 : static_cast<long>(e) * H + n0, I, lane, layout);
  u32x4 b[KSMAX];
#pragma unroll
  for (int s = 0; s < KSMAX; ++s) b[s] = ld_kstep<GUARD>(rd, s, KS);

  for (int mt = 0; mt * 16 < m; ++mt) {
    if (mt > 0) {
      const int r = mt * 16 + c;
      ra = clamp_row(pair_rows[off + (r < m ? r : 0)], P);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = mt * 16 + 4 * g + q;
        ro[q] = clamp_row(pair_rows[off + (rr < m ? rr : 0)], P);
      }
    }
    const bool ok = mt * 16 + c < m;
    const uint16_t* ar = act + static_cast<size_t>(ra) * I + g * 8;
    u32x4 a[KSMAX];
#pragma unroll
    for (int s = 0; s < KSMAX; ++s) {
      const u32x4 v = ld16(ar + (GUARD ? (s < KS ? s : 0) : s) * 32);
      a[s] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSMAX; ++s) acc = mfma_bf16(a[s], b[s], acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = mt * 16 + 4 * g + q;
      if (rr < m) ypair[static_cast<size_t>(ro[q]) * H + n0 + c] = acc[q];
    }
  }
}

// ---- many tokens per group (multi-block batches) ---------------------------
// With many blocks in one call a touched expert serves tens of tokens, and a
// work item (one slot: at most kSlotChunk = 64 tokens) holds all of them as
// four 16-token MFMA row tiles.  Every weight byte is still read once per
// slot, straight into registers, while the token rows are read once per
// work item (not once per 16 weight rows).  A group of more than 64 tokens
// is split into sibling slots; their weight loads go through the caches and
// the siblings run side by side on one XCD, so the repeated reads mostly
// hit L2.  At H = 2048 the per-element arithmetic is that of the kernels
// above (8 k-steps per wave in both, partials summed in wave order), so the
// results are bit-identical to theirs; at smaller H the K split differs (a
// wave's slice is H/256 k-steps here, 8 there).
#ifndef BDM_WIDE_GU_GROUPS
#define BDM_WIDE_GU_GROUPS 8           // from kWideGuBigT tokens; 4 below
#endif
#ifndef BDM_WIDE_GU_BIG_T
#define BDM_WIDE_GU_BIG_T 512
#endif
#ifndef BDM_WIDE_GU_SMALL_GROUPS
#define BDM_WIDE_GU_SMALL_GROUPS 4     // column groups per gate/up item below BDM_WIDE_GU_BIG_T
#endif
#ifndef BDM_WIDE_DN_GROUPS
#define BDM_WIDE_DN_GROUPS 1
#endif
#ifndef BDM_WIDE_XCD
#define BDM_WIDE_XCD 1
#endif
#ifndef BDM_WIDE_REUSE
#define BDM_WIDE_REUSE 1
#endif
#ifndef BDM_GU_TILE_SKIP
#define BDM_GU_TILE_SKIP 1
#endif
// weight loads of the many-token kernels: through the caches when another
// slot reads the same weights (TEMP), else streamed
template <bool TEMP>
__device__ __forceinline__ u32x4 ld16_w(const void* p) {
  if constexpr (TEMP && BDM_WIDE_REUSE) return ld16(p);
  else return ld16_stream(p);
}
constexpr int kWideMt = 4;                             // 16-token row tiles per work item
constexpr int kWideGuGroups = BDM_WIDE_GU_GROUPS;      // 16-column groups of I per gate/up item
constexpr int kWideGuBigT = BDM_WIDE_GU_BIG_T;         // (fewer slots below: 4 groups, more items)
constexpr int kWideDnGroups = BDM_WIDE_DN_GROUPS;      // 16-row groups of H per wave in down

// gate/up: work item = (slot, gpi column groups).  The 8 waves
// split K = H (KSW k-steps each) and hold their K-slice of the slot's token
// rows in registers; the weights stream one 16-row group at a time,
// alternating gate and up, and each k-step of a matrix's next group is
// requested as soon as the current one has been multiplied.  The 8 partial
// products of a group meet in LDS (double-buffered, one barrier per group)
// and are summed in wave order; silu(g) * u is stored as bf16.
template <int KSW, bool TEMP>
__device__ __forceinline__ void gateup_wide_item(
    float (*part)[2][kGuWaves][kWideMt][4][kWave], int* srow, const int4 slot, int run, int gpi,
    const uint16_t* __restrict__ x, int H, int I, int E, int k, int P, int layout,
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ ws_gate, const uint16_t* __restrict__ ws_up,
    const int32_t* __restrict__ pair_rows, uint16_t* __restrict__ act) {
  constexpr int MT = kWideMt;
  const int ngi = I / 16;                                 // column groups of I
  const int e = slot.x;
  const int off = slot.y;
  const int m = slot.z < 16 * MT ? slot.z : 16 * MT;
  const int q0 = run * gpi;                               // first column group
  const int nq = (ngi - q0) < gpi ? (ngi - q0) : gpi;
  const int K1 = k + 1;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int s0 = wave * KSW;

  const uint16_t* wg = e == E ? ws_gate : w_gate;
  const uint16_t* wu = e == E ? ws_up : w_up;
  const long wrow = (e == E) ? 0 : static_cast<long>(e) * I;
  // weights of column group q of this run; q >= nq: 16 bytes of token row
  // 0 per lane instead (valid, cached, ignored)
  auto load = [&](const uint16_t* W, int q, u32x4(&b)[KSW]) {
    const FragPtr f = q < nq ? frag_ptr_gu(W, wrow + 16L * (q0 + q), H, lane, layout)
                             : FragPtr{x + c * 8, 0};
#pragma unroll
    for (int s = 0; s < KSW; ++s) b[s] = ld16_w<TEMP>(f.p + (s0 + s) * f.step);
  };
  // pair rows first, then the weight burst (in-order completion: the rows
  // can be waited for without waiting for the weights)
  const int prow = tid < 16 * MT ? clamp_row(pair_rows[off + (tid < m ? tid : 0)], P) : 0;
  u32x4 bg[KSW], bu[KSW];
  load(wg, 0, bg);
  load(wu, 0, bu);
  if (tid < 16 * MT) srow[tid] = prow;
  __syncthreads();
  // this wave's K-slice of the slot's token rows (rows >= m are zero; a
  // tile wholly past m loads nothing, a workgroup-uniform test)
  u32x4 a[MT][KSW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (!BDM_GU_TILE_SKIP || 16 * mt < m) {
      const int r = 16 * mt + c;
      const bool ok = r < m;
      const uint16_t* xr = x + static_cast<size_t>(srow[r] / K1) * H + g * 8;
#pragma unroll
      for (int s = 0; s < KSW; ++s) {
        const u32x4 v = ld16(xr + (s0 + s) * 32);
        a[mt][s] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int s = 0; s < KSW; ++s) a[mt][s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // the partial products of one matrix's group; each k-step of the same
  // matrix's next group is requested as soon as this one has been used
  auto partial = [&](u32x4(&b)[KSW], const uint16_t* W, int qn, float* pp) {
    const FragPtr fn = qn < nq ? frag_ptr_gu(W, wrow + 16L * (q0 + qn), H, lane, layout)
                               : FragPtr{x + c * 8, 0};
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(a[mt][s], b[s], acc[mt]);
      b[s] = ld16_w<TEMP>(fn.p + (s0 + s) * fn.step);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[(mt * 4 + i) * kWave + lane] = acc[mt][i];
  };
  for (int q = 0; q < nq; ++q) {
    const int buf = q & 1;
    partial(bg, wg, q + 1, &part[0][buf][wave][0][0][0]);
    partial(bu, wu, q + 1, &part[1][buf][wave][0][0][0]);
    __syncthreads();
    // fold: 64 tokens x 16 columns, two per thread; thread o reads element
    // (mt, i, lane ln) of every wave's partials, consecutive threads
    // consecutive lanes (no bank conflicts): token 16 mt + 4 (ln / 16) + i,
    // column ln % 16
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int o = tid + f * kGuWaves * kWave;
      const int ln = o & 63, i = (o >> 6) & 3, mt = o >> 8;
      const int r = 16 * mt + 4 * (ln >> 4) + i, cc = ln & 15;
      float gs = part[0][buf][0][mt][i][ln], us = part[1][buf][0][mt][i][ln];
#pragma unroll
      for (int w = 1; w < kGuWaves; ++w) {
        gs += part[0][buf][w][mt][i][ln];
        us += part[1][buf][w][mt][i][ln];
      }
      if (r < m) {
        const float av = gs / (1.0f + expf(-gs)) * us;
        act[static_cast<size_t>(srow[r]) * I + 16 * (q0 + q) + cc] = f32_to_bf16(av);
      }
    }
  }
}

template <int KSW>
__global__ __launch_bounds__(kGuWaves * 64, 1) void gateup_wide_kernel(
    const uint16_t* __restrict__ x, int H, int I, int E, int k, int P, int layout,
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ ws_gate, const uint16_t* __restrict__ ws_up,
    const int4* __restrict__ slots, const int32_t* __restrict__ pair_rows,
    const int32_t* __restrict__ info, int nslots, int gpi, uint16_t* __restrict__ act) {
  static_assert(kGuWaves == 8, "8 waves split K");
  __shared__ float part[2][2][kGuWaves][kWideMt][4][kWave];   // [gate/up][buffer]: 128 KB
  __shared__ int srow[16 * kWideMt];

  const int runs = (I / 16 + gpi - 1) / gpi;
  int si, run;
  if (BDM_WIDE_XCD) {
    // workgroup b runs on XCD b % 8: XCD x takes items [x Q, x Q + Q) of
    // the n slots x runs items in run-major order, so the chunks of one
    // expert's column run are adjacent, on one XCD, at the same time
    int n = info[0];
    n = n < 0 ? 0 : (n > nslots ? nslots : n);
    const int N = n * runs;
    const int Q = (N + 7) / 8;
    const int ii = static_cast<int>(blockIdx.x) / 8;
    const int w = static_cast<int>(blockIdx.x % 8) * Q + ii;
    if (ii >= Q || w >= N) return;
    si = w % n;
    run = w / n;
  } else {
    si = blockIdx.x / runs;
    run = blockIdx.x % runs;
  }
  const int4 slot = slots[si];
  // past the touched groups (-1), or a slot that is not a valid group
  if (!slot_ok(slot.x, slot.y, slot.z, E, P, ws_gate != nullptr)) return;
  // a group split over several slots is read once per slot: those reads
  // go through the caches (the sibling slots run next to it), the others
  // stream
  if (slot.w > 1)
    gateup_wide_item<KSW, true>(part, srow, slot, run, gpi, x, H, I, E, k, P, layout, w_gate,
                                w_up, ws_gate, ws_up, pair_rows, act);
  else
    gateup_wide_item<KSW, false>(part, srow, slot, run, gpi, x, H, I, E, k, P, layout, w_gate,
                                 w_up, ws_gate, ws_up, pair_rows, act);
}

// down: work item = (slot, 8 waves x kWideDnGroups groups of 16 rows of H).
// The slot's activation rows are staged once in LDS in MFMA operand order
// (tile (mt, s) = 64 lanes x 16 B, conflict-free reads); every wave then
// owns its own 16-row groups over the whole K = I, each k-step of its next
// group requested as soon as the current one has been multiplied, and
// stores fp32 results per (token, slot) row.
#ifndef BDM_DN_STAGE_SKIP
#define BDM_DN_STAGE_SKIP 1
#endif
#ifndef BDM_DN_WIDE_WAVES_PER_EU
#define BDM_DN_WIDE_WAVES_PER_EU 4     // two workgroups per CU (<= 128 registers)
#endif
template <int KSMAX, bool TEMP>
__device__ __forceinline__ void down_wide_item(
    u32x4 (*at)[KSMAX][kWave], int* srow, const int4 slot, int run,
    const uint16_t* __restrict__ act, int H, int I, int E, int P, int layout,
    const uint16_t* __restrict__ w_down, const uint16_t* __restrict__ ws_down,
    const int32_t* __restrict__ pair_rows, float* __restrict__ ypair) {
  constexpr int MT = kWideMt;
  constexpr int NW = 8;
  const int ngh = H / 16;
  const int per = NW * kWideDnGroups;                  // groups per work item
  const int e = slot.x;
  const int off = slot.y;
  const int m = slot.z < 16 * MT ? slot.z : 16 * MT;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int KS = I / 32;
  const int gbase = run * per + wave * kWideDnGroups;

  const uint16_t* W = e == E ? ws_down : w_down;
  const long wrow = (e == E) ? 0 : static_cast<long>(e) * H;
  // weights of this wave's group j; past its groups (or past H): 16 bytes of
  // activation row 0 per lane instead (valid, cached, ignored)
  auto wptr = [&](int j) -> FragPtr {
    const int gi = gbase + j;
    return (j < kWideDnGroups && gi < ngh) ? frag_ptr(W, wrow + 16L * gi, I, lane, layout)
                                           : FragPtr{act + c * 8, 0};
  };
  auto ldk = [&](FragPtr f, int s) -> u32x4 {
    const bool on = s < KS;
    const u32x4 v = ld16_w<TEMP>(f.p + (on ? s : 0) * f.step);
    return on ? v : u32x4{0u, 0u, 0u, 0u};
  };
  const int prow = tid < 16 * MT ? clamp_row(pair_rows[off + (tid < m ? tid : 0)], P) : 0;
  u32x4 b[KSMAX];
  {
    const FragPtr f = wptr(0);
#pragma unroll
    for (int s = 0; s < KSMAX; ++s) b[s] = ldk(f, s);
  }
  if (tid < 16 * MT) srow[tid] = prow;
  __syncthreads();
  // stage the activation rows: chunk ch -> tile (mt, s) = ch / 64, lane
  // l = ch % 64 holding row 16 mt + l % 16, values 8 (l / 16) .. +7 of
  // k-step s (consecutive threads write consecutive 16 bytes: no bank
  // conflicts); all loads of a batch first
  constexpr int NCH = 16 * MT * KSMAX * 4 / (NW * kWave);
  static_assert(NCH * NW * kWave == 16 * MT * KSMAX * 4, "whole chunks per thread");
  constexpr int NB = NCH >= 4 ? 4 : NCH;           // chunks per batch
  static_assert(NCH % NB == 0, "whole batches");
#pragma unroll
  for (int u0 = 0; u0 < NCH; u0 += NB) {
    u32x4 v[NB];
    // a batch whose rows all lie past the slot's tokens stores zeros only
    // (workgroup-uniform)
    const bool live = !BDM_DN_STAGE_SKIP || 16 * ((u0 * NW * kWave / 64) / KSMAX) < m;
    if (live) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int ch = tid + (u0 + u) * NW * kWave;
        const int l = ch & 63, s = (ch >> 6) % KSMAX, r = 16 * ((ch >> 6) / KSMAX) + (l & 15);
        v[u] = ld16(act + static_cast<size_t>(srow[r]) * I + (s < KS ? s : 0) * 32 +
                    (l >> 4) * 8);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NB; ++u) v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int ch = tid + (u0 + u) * NW * kWave;
      const int l = ch & 63, s = (ch >> 6) % KSMAX, r = 16 * ((ch >> 6) / KSMAX) + (l & 15);
      at[r >> 4][s][l] = (r < m && s < KS) ? v[u] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // each k-step of the next group is requested as soon as this group's
  // k-step has been multiplied (one group per wave in flight, in order)
  for (int j = 0; j < kWideDnGroups; ++j) {
    const FragPtr fn = wptr(j + 1);
    // an opaque zero: the operand reads stay inside the loop (hoisted out,
    // the 64 tiles would take 256 registers)
    int lz = lane;
    asm volatile("" : "+v"(lz));
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSMAX; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(at[mt][s][lz], b[s], acc[mt]);
      b[s] = ldk(fn, s);
    }
    const int gi = gbase + j;
    if (gi < ngh) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * g + i;
          if (r < m) ypair[static_cast<size_t>(srow[r]) * H + 16 * gi + c] = acc[mt][i];
        }
    }
  }
}

template <int KSMAX>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(
    BDM_DN_WIDE_WAVES_PER_EU, BDM_DN_WIDE_WAVES_PER_EU))) void down_wide_kernel(
    const uint16_t* __restrict__ act, int H, int I, int E, int P, int layout,
    const uint16_t* __restrict__ w_down, const uint16_t* __restrict__ ws_down,
    const int4* __restrict__ slots, const int32_t* __restrict__ pair_rows,
    float* __restrict__ ypair) {
  __shared__ u32x4 at[kWideMt][KSMAX][kWave];          // 64 KB at KSMAX = 16
  __shared__ int srow[16 * kWideMt];
  // item b = (slot b / runs, run b % runs): with 16 runs (H = 2048) run r of
  // every slot lands on XCD r % 8, so sibling slots of one group meet there
  const int runs = (H / 16 + 8 * kWideDnGroups - 1) / (8 * kWideDnGroups);
  const int4 slot = slots[blockIdx.x / runs];
  if (!slot_ok(slot.x, slot.y, slot.z, E, P, ws_down != nullptr)) return;
  const int run = blockIdx.x % runs;
  if (slot.w > 1)
    down_wide_item<KSMAX, true>(at, srow, slot, run, act, H, I, E, P, layout, w_down, ws_down,
                                pair_rows, ypair);
  else
    down_wide_item<KSMAX, false>(at, srow, slot, run, act, H, I, E, P, layout, w_down, ws_down,
                                 pair_rows, ypair);
}

// One workgroup per token; a thread owns 8 consecutive columns and issues all
// of its k+1 row loads before summing them in slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ypair, int H,
                                                      int k, int has_shared,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const float* __restrict__ topk_w,
                                                      const uint16_t* residual, uint16_t* y,
                                                      uint16_t* y_norm) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int h0 = threadIdx.x * 8;
  const bool on = h0 < H;
  if (!on && !y_norm) return;
  const int K1 = k + 1;
  const float* yrow = ypair + static_cast<size_t>(t) * K1 * H + (on ? h0 : 0);
  // every row load first (a slot the block coreset selector left empty, id
  // -1, has a row in the workspace that is loaded and then ignored)
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
    const u32x4 r = ld16(residual + static_cast<size_t>(t) * H + (on ? h0 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __uint_as_float(r[i] << 16);
      acc[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  }
  uint32_t used = 0u;
#pragma unroll
  for (int j = 0; j < BDM_MAX_TOPK; ++j)
    if (j < k) used |= (topk_idx[t * k + j] >= 0 ? 1u : 0u) << j;
#pragma unroll
  for (int j = 0; j <= BDM_MAX_TOPK; ++j) {
    const float yv[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w,
                         v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
    if (j < k && ((used >> j) & 1u)) {
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
  if (!on) o = u32x4{0u, 0u, 0u, 0u};
  if (y_norm) {
    // the next layer's RMSNorm of this row (eps 1e-6, unit gamma), the same
    // arithmetic as the RMSNorm kernel on the stored bf16 values
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(o[j] << 16);
      v[2 * j + 1] = __uint_as_float(o[j] & 0xffff0000u);
    }
    const float r = row_rms_scale(v, 1e-6f, H, part);
    if (on) {
      u32x4 q;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[j] = static_cast<uint32_t>(f32_to_bf16(v[2 * j] * r)) |
               (static_cast<uint32_t>(f32_to_bf16(v[2 * j + 1] * r)) << 16);
      *reinterpret_cast<u32x4*>(y_norm + static_cast<size_t>(t) * H + h0) = q;
    }
  }
  if (on) *reinterpret_cast<u32x4*>(y + static_cast<size_t>(t) * H + h0) = o;
}

void launch_experts(const uint16_t* x, int T, int H, int I, int E, int k, int has_shared,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                    const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                    const MoeMeta& meta, int layout, hipStream_t s) {
  // down reads its own matrices, packed the plain way in the gate/up pair layout
  const int dl = layout == BDM_LAYOUT_MFMA_TILES_GU ? BDM_LAYOUT_MFMA_TILES : layout;
  // upper bound on the slots; workgroups past the actual list exit at once
  const int groups = moe_max_slots(T, E, k, has_shared);
  const int P = T * (k + 1);
  const dim3 gu(groups * (I / kGuCols)), dn(groups * ((H + kDnRows - 1) / kDnRows));
  const int KS = H / 32;
  const int KI = I / 32;
// many-token kernels from 8 blocks: a skewed 8-block batch (its hottest
// experts take ~250 tokens, four 64-token slots) runs 20% faster on them, an
// even one 2% slower
#ifndef BDM_WIDE_MIN_T
#define BDM_WIDE_MIN_T 256
#endif
  const int ksw = H / 256;
  if (T >= BDM_WIDE_MIN_T && H % 256 == 0 && (ksw == 1 || ksw == 2 || ksw == 4 || ksw == 8) &&
      KI <= 16) {
    // fewer tokens, fewer slots: narrower gate/up items keep every CU busy
    const int gpi = T >= kWideGuBigT ? kWideGuGroups : BDM_WIDE_GU_SMALL_GROUPS;
    const int gu_runs = (I / 16 + gpi - 1) / gpi;
    const int dn_runs = (H / 16 + 8 * kWideDnGroups - 1) / (8 * kWideDnGroups);
    using GuWide = void (*)(const uint16_t*, int, int, int, int, int, int, const uint16_t*,
                            const uint16_t*, const uint16_t*, const uint16_t*, const int4*,
                            const int32_t*, const int32_t*, int, int, uint16_t*);
    const GuWide guw = ksw == 1   ? &gateup_wide_kernel<1>
                       : ksw == 2 ? &gateup_wide_kernel<2>
                       : ksw == 4 ? &gateup_wide_kernel<4>
                                  : &gateup_wide_kernel<8>;
    // (the XCD mapping needs every (XCD, index) pair up to ceil(items / 8))
    const int gu_grid = BDM_WIDE_XCD ? (groups * gu_runs + 7) / 8 * 8 : groups * gu_runs;
    guw<<<gu_grid, kGuWaves * 64, 0, s>>>(x, H, I, E, k, P, layout, w_gate, w_up, ws_gate,
                                          ws_up, meta.slots, meta.pair_rows, meta.info, groups,
                                          gpi, meta.act);
    down_wide_kernel<16><<<groups * dn_runs, 512, 0, s>>>(meta.act, H, I, E, P, dl, w_down,
                                                          ws_down, meta.slots, meta.pair_rows,
                                                          meta.ypair);
    combine_kernel<<<T, 256, 0, s>>>(meta.ypair, H, k, has_shared, meta.topk_idx, meta.topk_w,
                                     residual, y, y_norm);
    return;
  }
  if (KS == kGuWaves * 8) {
    gateup_kernel<8, false><<<gu, kGuWaves * 64, 0, s>>>(x, H, I, E, k, P, layout, w_gate, w_up, ws_gate,
                                                        ws_up, meta.slots, meta.pair_rows,
                                                        meta.act);
  } else {
    gateup_kernel<8, true><<<gu, kGuWaves * 64, 0, s>>>(x, H, I, E, k, P, layout, w_gate, w_up, ws_gate,
                                                       ws_up, meta.slots, meta.pair_rows,
                                                       meta.act);
  }
  if (KI == 16) {
    down_kernel<16, false><<<dn, kDnWaves * 64, 0, s>>>(meta.act, H, I, E, P, dl, w_down, ws_down, meta.slots,
                                              meta.pair_rows, meta.ypair);
  } else if (KI < 16) {
    down_kernel<16, true><<<dn, kDnWaves * 64, 0, s>>>(meta.act, H, I, E, P, dl, w_down, ws_down, meta.slots,
                                             meta.pair_rows, meta.ypair);
  } else {
    down_kernel<32, true><<<dn, kDnWaves * 64, 0, s>>>(meta.act, H, I, E, P, dl, w_down, ws_down, meta.slots,
                                             meta.pair_rows, meta.ypair);
  }
  combine_kernel<<<T, 256, 0, s>>>(meta.ypair, H, k, has_shared, meta.topk_idx, meta.topk_w,
                                   residual, y, y_norm);
}

BDM_DEBUG_WORD_READER(debug_words_experts)

}  // namespace bdm
