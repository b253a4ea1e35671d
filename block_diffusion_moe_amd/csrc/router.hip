// Router, top-k selection and token permutation for the routed MoE layer.
//
// Page "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second,
// read from its files", section "What Clover is": 256 routed experts, each
// token routed to 8 of them, plus one shared expert that is always on.
// Section "The expert selection": a block reads the union of its tokens'
// expert sets, so after routing the (token, expert) pairs are regrouped by
// expert and the experts actually touched are listed once.
//
// Two kernels:
//   router_logits_kernel  l[t][e] = x_t . w_router[e] (+ bias[e]), fp32.  One
//                         wave per expert row streams that row once and
//                         forms all T dot products (x stays in L2).
//   route_select_kernel   one workgroup: per-token softmax / top-k / weights
//                         (one wave per token, wave-wide argmax reductions),
//                         then the per-expert token bitmap in LDS, expert
//                         counts, offsets, the touched-expert list and the
//                         expert-grouped pair list.
#include "device.hpp"
#include "internal.hpp"

namespace bdm {

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x, int T,
                                                            int H, const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int E,
                                                            float* __restrict__ logits) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  // lane handles 8-element chunks c = lane, lane + 64, ... (H % 64 == 0)
  constexpr int kMaxChunks = BDM_MAX_HIDDEN_ / 512;  // chunks per lane at most
  const int nchunk = H / 8;
  float w[kMaxChunks][8];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) {
      const float4* p = reinterpret_cast<const float4*>(wr + static_cast<size_t>(e) * H + c * 8);
      const float4 lo = p[0], hi = p[1];
      w[i][0] = lo.x; w[i][1] = lo.y; w[i][2] = lo.z; w[i][3] = lo.w;
      w[i][4] = hi.x; w[i][5] = hi.y; w[i][6] = hi.z; w[i][7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[i][j] = 0.0f;
    }
  }
  const float b = bias ? bias[e] : 0.0f;
  for (int t = 0; t < T; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        const u32x4 v = ld16(x + static_cast<size_t>(t) * H + c * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(__uint_as_float(v[j] << 16), w[i][2 * j], acc);
          acc = fmaf(__uint_as_float(v[j] & 0xffff0000u), w[i][2 * j + 1], acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[static_cast<size_t>(t) * E + e] = acc + b;
  }
}

// Wave-wide argmax over (value, id): larger value wins, equal values keep the
// lower id.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oid = __shfl_xor(id, o, kWave);
    if (ov > v || (ov == v && oid < id)) {
      v = ov;
      id = oid;
    }
  }
}

__global__ __launch_bounds__(1024) void route_select_kernel(const float* __restrict__ logits,
                                                            int T, int E, int k, int renorm,
                                                            int has_shared, MoeMeta meta,
                                                            int32_t* __restrict__ user_idx,
                                                            float* __restrict__ user_w) {
  extern __shared__ uint32_t lds[];
  const int W32 = (T + 31) / 32;
  uint32_t* bitmap = lds;                      // [E][W32]
  int* counts = reinterpret_cast<int*>(bitmap + E * W32);   // [E + 1]
  int* offs = counts + (E + 1);                // [E + 2]
  int* scan_tmp = offs + (E + 2);              // [32]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int nwaves = blockDim.x / kWave;

  for (int i = tid; i < E * W32; i += blockDim.x) bitmap[i] = 0u;
  __syncthreads();

  // ---- per-token softmax, top-k, weights -------------------------------
  constexpr int kPer = BDM_MAX_EXPERTS_ / kWave;   // logits per lane at most
  const int per = (E + kWave - 1) / kWave;
  for (int t = wave; t < T; t += nwaves) {
    float v[kPer];
    const float* row = logits + static_cast<size_t>(t) * E;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + kWave * i;
      const float l = (i < per && e < E) ? row[e] : -INFINITY;
      v[i] = (l == l) ? l : -INFINITY;           // NaN logits rank last
    }
    uint32_t picked = 0u;
    float sel_v = 0.0f, first_v = 0.0f;
    int sel_e = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = INT32_MAX;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + kWave * i;
        if (i < per && e < E && !(picked & (1u << i))) {
          if (v[i] > bv || (v[i] == bv && e < be)) {
            bv = v[i];
            be = e;
          }
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
    // weights: exp(l_j - l_max) / sum over the picks (renorm) or over all E
    float z = (lane < k) ? expf(sel_v - first_v) : 0.0f;
    float den;
    if (renorm) {
      den = wave_sum(z);
    } else {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + kWave * i;
        if (i < per && e < E) s += expf(v[i] - first_v);
      }
      den = wave_sum(s);
    }
    if (lane < k) {
      const float w = z / den;
      meta.topk_idx[t * k + lane] = sel_e;
      meta.topk_w[t * k + lane] = w;
      if (user_idx) user_idx[t * k + lane] = sel_e;
      if (user_w) user_w[t * k + lane] = w;
      atomicOr(&bitmap[sel_e * W32 + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();

  // ---- counts per expert (group E = the shared expert, all T tokens) ----
  for (int e = tid; e <= E; e += blockDim.x) {
    int c = 0;
    if (e < E) {
      for (int w = 0; w < W32; ++w) c += __popc(bitmap[e * W32 + w]);
    } else {
      c = has_shared ? T : 0;
    }
    counts[e] = c;
  }
  __syncthreads();

  // ---- exclusive scan of counts -> offs; touched list ------------------
  // Serial over the waves' partial sums: E + 1 <= 1025 entries, two passes of
  // 1024 threads at most.  The touched list puts the shared expert first,
  // then every routed expert with tokens in increasing id.
  int carry_off = 0;
  int carry_tch = has_shared ? 1 : 0;
  for (int base = 0; base <= E; base += blockDim.x) {
    const int e = base + tid;
    const int c = (e <= E) ? counts[e] : 0;
    const int f = (e < E && c > 0) ? 1 : 0;
    // inclusive wave scans of c and f
    int sc = c, sf = f;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int oc = __shfl_up(sc, o, kWave);
      const int of = __shfl_up(sf, o, kWave);
      if (lane >= o) {
        sc += oc;
        sf += of;
      }
    }
    if (lane == kWave - 1) {
      scan_tmp[wave] = sc;
      scan_tmp[16 + wave] = sf;
    }
    __syncthreads();
    int wc = 0, wf = 0;
    for (int w = 0; w < wave; ++w) {
      wc += scan_tmp[w];
      wf += scan_tmp[16 + w];
    }
    const int off = carry_off + wc + sc - c;
    const int pos = carry_tch + wf + sf - f;
    if (e <= E) offs[e] = off;
    if (f) meta.touched[pos] = e;
    int tot_c = 0, tot_f = 0;
    for (int w = 0; w < nwaves; ++w) {
      tot_c += scan_tmp[w];
      tot_f += scan_tmp[16 + w];
    }
    __syncthreads();
    carry_off += tot_c;
    carry_tch += tot_f;
  }
  if (tid == 0) {
    offs[E + 1] = carry_off;
    if (has_shared) meta.touched[0] = E;
    meta.info[0] = carry_tch;      // number of touched groups (shared included)
    meta.info[1] = carry_off;      // number of (token, expert) pairs
  }
  __syncthreads();
  for (int e = tid; e <= E + 1; e += blockDim.x) meta.offs[e] = offs[e];

  // ---- pair list: group e holds its tokens in increasing order ----------
  const int K1 = k + 1;
  for (int p = tid; p < T * k; p += blockDim.x) {
    const int t = p / k;
    const int j = p - t * k;
    const int e = meta.topk_idx[p];
    int rank = 0;
    const uint32_t* bm = bitmap + e * W32;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(bm[w]);
    rank += __popc(bm[t >> 5] & ((1u << (t & 31)) - 1u));
    const int pos = offs[e] + rank;
    meta.pair_token[pos] = t;
    meta.pos[t * K1 + j] = pos;
  }
  if (has_shared) {
    for (int t = tid; t < T; t += blockDim.x) {
      const int pos = offs[E] + t;
      meta.pair_token[pos] = t;
      meta.pos[t * K1 + k] = pos;
    }
  }
}

size_t route_select_lds_bytes(int T, int E) {
  const int W32 = (T + 31) / 32;
  return sizeof(uint32_t) * (static_cast<size_t>(E) * W32 + (E + 1) + (E + 2) + 32);
}

void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, const MoeMeta& meta, int32_t* user_idx,
                   float* user_w, hipStream_t s) {
  router_logits_kernel<<<(E + 3) / 4, 256, 0, s>>>(x, T, H, wr, bias, E, meta.logits);
  route_select_kernel<<<1, 1024, route_select_lds_bytes(T, E), s>>>(
      meta.logits, T, E, k, renorm, has_shared, meta, user_idx, user_w);
}

}  // namespace bdm
