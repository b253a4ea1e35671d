// Internal declarations shared by the translation units of libbdmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bdmoe.h"

#define BDM_MAX_HIDDEN_ BDM_MAX_HIDDEN
#define BDM_MAX_EXPERTS_ BDM_MAX_EXPERTS

namespace bdm {

// Views into the MoE workspace (all device pointers).  Sizes for T tokens,
// E routed experts, k picks, P = T*k (+T with a shared expert) pairs.
struct MoeMeta {
  float* logits;        // [T][E]     router logits (fp32)
  int32_t* topk_idx;    // [T][k]     picks, decreasing weight
  float* topk_w;        // [T][k]     their weights
  int32_t* info;        // [4]        [0] touched groups, [1] pairs
  int32_t* offs;        // [E+2]      group start in the pair list; group E = shared
  int32_t* touched;     // [E+1]      touched groups, shared first
  int32_t* pair_token;  // [P]        token of each pair, grouped by expert
  int32_t* pos;         // [T][k+1]   pair index of (t, j); j = k is the shared expert
  uint16_t* act;        // [P][I]     bf16 SwiGLU activations per pair
  float* ypair;         // [P][H]     fp32 expert outputs per pair
};

size_t route_select_lds_bytes(int T, int E);

void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, const MoeMeta& meta, int32_t* user_idx,
                   float* user_w, hipStream_t s);

void launch_experts(const uint16_t* x, int T, int H, int I, int E, int k, int has_shared,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                    const uint16_t* residual, uint16_t* y, const MoeMeta& meta, hipStream_t s);

// Head: partial softmax statistics per (token, vocabulary tile).
constexpr int kHeadTileRows = 256;   // vocabulary rows per workgroup
constexpr int kHeadTokChunk = 32;    // tokens per head pass

struct HeadParts {
  float* m;     // [T][ntiles]
  float* s;     // [T][ntiles]
  int32_t* a;   // [T][ntiles]
};

void launch_head(const uint16_t* h, int T, int H, const uint16_t* w, int V, int32_t mask_id,
                 float threshold, int fallback, int32_t* tokens, int32_t* argmax, float* conf,
                 int32_t* n_committed, const HeadParts& parts, hipStream_t s);

void launch_rmsnorm(const uint16_t* x, const float* gamma, float eps, int T, int H,
                    uint16_t* out, hipStream_t s);

}  // namespace bdm
