// Device helpers shared by the gfx950 kernels of libbdmoe.
//
// MFMA used throughout: v_mfma_f32_16x16x32_bf16 (one wave64 computes a
// 16x16 fp32 tile from a 16x32 bf16 A tile and a 32x16 bf16 B tile).
// Register layout, lane l = 16*g + c (c = l % 16, g = l / 16):
//   A operand  (8 x bf16 per lane): row c,    k = 8*g + 0..7
//   B operand  (8 x bf16 per lane): column c, k = 8*g + 0..7
//   C/D        (4 x fp32 per lane): column c, rows 4*g + 0..3
// The kernels only rely on A and B using the same k <-> (g, item) map, so a
// lane's 8 consecutive k values are one 16-byte load from a row-major
// (k-contiguous) operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdmoe.h"

namespace bdm {

// ---- bounds checks of data-dependent indices ------------------------------
// An index read from memory (a slot of the table, a pair row, a pick, a
// token id) or derived from one is passed through chk(i, n, code) before it
// addresses a buffer of n elements.  In the debug build (BDM_DEBUG_BOUNDS=1,
// libbdmoe_debug.so) an index outside [0, n) sets bit `code` of this source
// file's violation word and is clamped into range, so the access stays in
// its buffer and the call completes; bdm_debug_bounds() reads and clears
// the words.  In the release build chk is the index itself.  Checks that a
// release kernel already makes (it clamps or skips) report through
// note_oob(code) in the debug build.
#ifndef BDM_DEBUG_BOUNDS
#define BDM_DEBUG_BOUNDS 0
#endif
enum BdmCheck : unsigned {
  kChkSlot = 0,       // a slot-table entry that is neither a valid group nor the end mark
  kChkPairRow = 1,    // a (token, slot) pair row outside [0, T (k+1))
  kChkExpert = 2,     // an expert id outside [0, E) (-1 = empty pick is allowed)
  kChkTokenRow = 3,   // a token row outside [0, T)
  kChkVocabRow = 4,   // a head / embedding row outside [0, V)
  kChkTokenId = 5,    // a token id outside [0, V) given to the embedding gather
  kChkStat = 6,       // an online-softmax partial outside [0, T * parts)
  kChkCand = 7,       // a re-route candidate or rank outside its table
  kChkWs = 8,         // a workspace table index outside its sized extent
};
#if BDM_DEBUG_BOUNDS
static __device__ unsigned int g_bdm_oob;
__device__ __forceinline__ void note_oob(unsigned code) { atomicOr(&g_bdm_oob, 1u << code); }
__device__ __forceinline__ long chk(long i, long n, unsigned code) {
  if (i >= 0 && i < n) return i;
  note_oob(code);
  return i < 0 || n <= 0 ? 0 : n - 1;
}
// Host side: read this file's violation word into *out and clear it.
#define BDM_DEBUG_WORD_READER(NAME)                                              \
  int NAME(unsigned int* out) {                                                  \
    unsigned int v = 0u;                                                         \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_bdm_oob), sizeof(v)) != hipSuccess) \
      return -1;                                                                 \
    const unsigned int z = 0u;                                                   \
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_bdm_oob), &z, sizeof(z)) != hipSuccess)   \
      return -1;                                                                 \
    *out |= v;                                                                   \
    return 0;                                                                    \
  }
#else
__device__ __forceinline__ void note_oob(unsigned) {}
__device__ __forceinline__ long chk(long i, long, unsigned) { return i; }
#define BDM_DEBUG_WORD_READER(NAME) \
  int NAME(unsigned int*) { return 0; }
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16-byte loads.  `ld16_stream` marks data read exactly once (expert and head
// weights) as non-temporal so it does not evict reused data from the caches.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// This lane's 16 bytes of k-step 0 of the 16 weight rows row0 .. row0+15 of a
// bf16 matrix with K columns, and the element stride from one k-step (32 k)
// to the next: row-major [R][K] (rows 4 KB apart at K = 2048) or the packed
// MFMA-tile layout (one contiguous 1 KB fragment per k-step, see pack.hip).
struct FragPtr {
  const uint16_t* p;
  int step;
};

__device__ __forceinline__ FragPtr frag_ptr(const uint16_t* W, long row0, int K, int lane,
                                            int layout) {
  if (layout == BDM_LAYOUT_MFMA_TILES)
    return {W + (row0 / 16) * (K / 32) * 512 + lane * 8, 512};
  return {W + (row0 + (lane & 15)) * K + (lane >> 4) * 8, 32};
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- cross-lane reductions on DPP (no LDS round trips) ---------------------
// Within a 16-lane row: xor 1 and xor 2 (quad permutes), then the half-row
// mirror (lane i <-> 7-i) and the row mirror (i <-> 15-i).  With a
// commutative combiner every lane of the row ends with the same value.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

template <class Op>
__device__ __forceinline__ float row_reduce_f(float v, Op op) {
  v = op(v, dpp_f<kDppXor1>(v));
  v = op(v, dpp_f<kDppXor2>(v));
  v = op(v, dpp_f<kDppHalfMirror>(v));
  v = op(v, dpp_f<kDppMirror>(v));
  return v;
}

// The four rows' results, combined in a fixed order on every lane.
template <class Op>
__device__ __forceinline__ float wave_reduce_f(float v, Op op) {
  v = row_reduce_f(v, op);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce_f(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ int wave_sum_i(int v) {
  auto add = [](int a, int b) { return a + b; };
  v = add(v, dpp_i<kDppXor1>(v));
  v = add(v, dpp_i<kDppXor2>(v));
  v = add(v, dpp_i<kDppHalfMirror>(v));
  v = add(v, dpp_i<kDppMirror>(v));
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce_f(v, [](float a, float b) { return fmaxf(a, b); });
}

// Wave-wide argmax over (value, id): larger value wins, equal values keep the
// lower id.  Every lane returns the winner.
__device__ __forceinline__ bool argmax_better(float ov, int oid, float v, int id) {
  return ov > v || (ov == v && oid < id);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& id) {
  const float ov = dpp_f<CTRL>(v);
  const int oid = dpp_i<CTRL>(id);
  if (argmax_better(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  argmax_step<kDppXor1>(v, id);
  argmax_step<kDppXor2>(v, id);
  argmax_step<kDppHalfMirror>(v, id);
  argmax_step<kDppMirror>(v, id);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bid = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int rid = __builtin_amdgcn_readlane(id, 16 * r);
    if (argmax_better(rv, rid, bv, bid)) {
      bv = rv;
      bid = rid;
    }
  }
  v = bv;
  id = bid;
}

// Online-softmax statistics of a set of logits: running max m, sum of
// exp(l - m), and the lowest index attaining m (INT32_MAX when empty).
struct SoftStat {
  float m;
  float s;
  int a;
};

__device__ __forceinline__ SoftStat softstat_empty() { return {-INFINITY, 0.0f, INT32_MAX}; }

// Associative merge; the winner is the larger max, equal maxima keep the
// lower index.  Deterministic for a fixed merge tree.
__device__ __forceinline__ SoftStat softstat_merge(SoftStat x, SoftStat y) {
  SoftStat r;
  r.m = fmaxf(x.m, y.m);
  if (r.m == -INFINITY) return {-INFINITY, 0.0f, min(x.a, y.a)};
  const float sx = (x.m == -INFINITY) ? 0.0f : x.s * expf(x.m - r.m);
  const float sy = (y.m == -INFINITY) ? 0.0f : y.s * expf(y.m - r.m);
  r.s = sx + sy;
  if (x.m > y.m) r.a = x.a;
  else if (y.m > x.m) r.a = y.a;
  else r.a = min(x.a, y.a);
  return r;
}

template <int CTRL>
__device__ __forceinline__ SoftStat dpp_stat(SoftStat v) {
  return {dpp_f<CTRL>(v.m), dpp_f<CTRL>(v.s), dpp_i<CTRL>(v.a)};
}

// Merge across the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ SoftStat row_merge_stat(SoftStat v) {
  v = softstat_merge(v, dpp_stat<kDppXor1>(v));
  v = softstat_merge(v, dpp_stat<kDppXor2>(v));
  v = softstat_merge(v, dpp_stat<kDppHalfMirror>(v));
  v = softstat_merge(v, dpp_stat<kDppMirror>(v));
  return v;
}

// Online statistics of a logit row for the verify epilogue: max m, s = sum
// exp(l - m), q = sum exp(l - m) (l - m) (entropy = log s - q / s), argmax a
// (lowest index on ties) and the candidate's logit lc (-inf until seen).
struct VStat {
  float m;
  float s;
  float q;
  int a;
  float lc;
};

__device__ __forceinline__ VStat vstat_empty() { return {-INFINITY, 0.0f, 0.0f, INT32_MAX, -INFINITY}; }

// Associative merge (deterministic for a fixed merge tree).  A side with
// m = -inf holds no element and contributes nothing.
__device__ __forceinline__ VStat vstat_merge(VStat x, VStat y) {
  VStat r;
  r.m = fmaxf(x.m, y.m);
  r.lc = fmaxf(x.lc, y.lc);
  if (r.m == -INFINITY) {
    r.s = 0.0f;
    r.q = 0.0f;
    r.a = min(x.a, y.a);
    return r;
  }
  float s = 0.0f, q = 0.0f;
  if (x.m != -INFINITY) {
    const float d = x.m - r.m, e = expf(d);
    s += x.s * e;
    q += e * (x.q + d * x.s);
  }
  if (y.m != -INFINITY) {
    const float d = y.m - r.m, e = expf(d);
    s += y.s * e;
    q += e * (y.q + d * y.s);
  }
  r.s = s;
  r.q = q;
  if (x.m > y.m) r.a = x.a;
  else if (y.m > x.m) r.a = y.a;
  else r.a = min(x.a, y.a);
  return r;
}

template <int CTRL>
__device__ __forceinline__ VStat dpp_vstat(VStat v) {
  return {dpp_f<CTRL>(v.m), dpp_f<CTRL>(v.s), dpp_f<CTRL>(v.q), dpp_i<CTRL>(v.a),
          dpp_f<CTRL>(v.lc)};
}

__device__ __forceinline__ VStat row_merge_vstat(VStat v) {
  v = vstat_merge(v, dpp_vstat<kDppXor1>(v));
  v = vstat_merge(v, dpp_vstat<kDppXor2>(v));
  v = vstat_merge(v, dpp_vstat<kDppHalfMirror>(v));
  v = vstat_merge(v, dpp_vstat<kDppMirror>(v));
  return v;
}

// RMSNorm scale of one row held as 8 consecutive fp32 values per thread
// (thread i: elements 8i .. 8i+7; threads past the row hold zeros) in a
// 256-thread workgroup: 1 / sqrt(mean(x^2) + eps), summed in a fixed order
// (per thread, DPP within the wave, then the 4 waves pairwise).  `part`: 4
// floats of LDS.  Every thread of the workgroup must call it.
__device__ __forceinline__ float row_rms_scale(const float (&v)[8], float eps, int H,
                                               float* part) {
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x % kWave) == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  return 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
}

}  // namespace bdm
