// Internal declarations shared by the translation units of libbdmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bdmoe.h"

#define BDM_MAX_HIDDEN_ BDM_MAX_HIDDEN
#define BDM_MAX_EXPERTS_ BDM_MAX_EXPERTS

// 1 in the bounds-checked debug build (libbdmoe_debug.so)
#ifndef BDM_DEBUG_BOUNDS
#define BDM_DEBUG_BOUNDS 0
#endif

namespace bdm {

// Views into the MoE workspace (all device pointers) for T tokens, E routed
// experts and k picks.  Rows of act / ypair are (token, slot) pairs: row
// t*(k+1)+j holds the j-th pick of token t, row t*(k+1)+k its shared expert.
constexpr int kRouterParts = 4;   // K-parts of the router GEMM (summed by select)
constexpr int kCoreCand = 32;     // ranked first-pass candidates per token (coreset selector)

// An expert work item serves at most kSlotChunk of its group's tokens; a
// longer group (the shared expert, or a routed expert of a many-block batch)
// takes several consecutive slots.  Upper bound on the slots of a T-token
// layer: one per touched routed expert (<= min(T*k, E)), plus at most
// floor(T*k / kSlotChunk) extra chunks over all routed experts (none unless
// T > kSlotChunk: an expert holds a token at most once), plus the shared
// expert's ceil(T / kSlotChunk).
#ifndef BDM_SLOT_CHUNK
#define BDM_SLOT_CHUNK 64
#endif
constexpr int kSlotChunk = BDM_SLOT_CHUNK;
__host__ __device__ inline int moe_max_slots(int T, int E, int k, int has_shared) {
  const int routed = T * k < E ? T * k : E;
  const int extra = T > kSlotChunk ? (T * k) / kSlotChunk : 0;
  const int shared = has_shared ? (T + kSlotChunk - 1) / kSlotChunk : 0;
  return routed + extra + shared;
}

struct MoeMeta {
  float* logits;        // [4][T][E]     partial router logits (fp32), one per K-part
  int32_t* topk_idx;    // [T][k]        picks, decreasing weight
  float* topk_w;        // [T][k]        their weights
  float* topk_p;        // [T][k]        first-pass probabilities (block coreset selector)
  int32_t* cand_id;     // [T][kCoreCand] first-pass candidates, ranked (coreset selector)
  float* cand_l;        // [T][kCoreCand] their logits
  int32_t* info;        // [4]           [0] number of touched expert groups
  int4* slots;          // [E+1]         {expert, offset, count, slots of the group} per slot, then -1
  int32_t* pair_rows;   // [T*(k+1)]     (token, slot) rows grouped by expert
  uint16_t* act;        // [T*(k+1)][I]  bf16 SwiGLU activations
  float* ypair;         // [T*(k+1)][H]  fp32 expert outputs
};

// top_p > 0: block coreset selector over blocks of `block` tokens (n_kept
// nullable, one count per block); top_p <= 0: plain top-k routing.  xn
// non-null: x is un-normalised, the router routes on RMSNorm(x) (eps 1e-6,
// unit gamma) and writes it to xn.
void launch_router(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                   int k, int renorm, int has_shared, float top_p, int block,
                   const MoeMeta& meta, int32_t* user_idx, float* user_w, int32_t* n_kept,
                   uint16_t* xn, hipStream_t s);

void launch_experts(const uint16_t* x, int T, int H, int I, int E, int k, int has_shared,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                    const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                    const MoeMeta& meta, int layout, hipStream_t s);

// Head: partial softmax statistics per (token, vocabulary tile).
constexpr int kHeadTokChunk = 32;    // tokens per head pass
#ifndef BDM_HEAD_WAVES
#define BDM_HEAD_WAVES 8
#endif
constexpr int kHeadWaves = BDM_HEAD_WAVES;   // waves per head workgroup

struct HeadParts {
  int grid;     // head workgroups (one per CU)
  float* m;     // [T][grid]
  float* s;     // [T][grid]
  int32_t* a;   // [T][grid]
};

size_t head_lds_bytes(int H);
int head_prepare();   // one-time kernel attribute set-up; 0 on success

void launch_head_stats(const uint16_t* h, int T, int H, const uint16_t* w, int V, int voff,
                       int layout, int32_t mask_id, float* pm, float* ps, int32_t* pa,
                       int pstride, int grid, hipStream_t s);

// n_left (nullable): masked rows that remain after the rule
// the commit rule is applied to every block of `block` rows on its own
// (block <= 0 or >= T: the whole call is one block)
void launch_unmask(const float* pm, const float* ps, const int32_t* pa, int T, int parts,
                   int pstride, int32_t mask_id, float threshold, int fallback, int block,
                   int32_t* tokens, int32_t* argmax, float* conf, int32_t* n_committed,
                   int32_t* n_left, hipStream_t s);

// x[t] = w_embed[tokens[t]] (ids clamped to [0, V)), bf16 rows of H, and
// xn = RMSNorm(x) (eps 1e-6, unit gamma; bit for bit the RMSNorm kernel)
void launch_embed(const int32_t* tokens, int T, const uint16_t* w_embed, int V, int H,
                  uint16_t* x, uint16_t* xn, hipStream_t s);

// the verify epilogue: statistics with the entropy term and the candidates'
// logits (H % 256 == 0), then the merge and the accept rule
void launch_head_verify_stats(const uint16_t* h, int T, int H, const uint16_t* w, int V,
                              int layout, const int32_t* cand, int ncand, float* pm, float* ps,
                              int32_t* pa, float* pq, float* plc, int pstride, int grid,
                              hipStream_t s);
void launch_verify_merge(const float* pm, const float* ps, const int32_t* pa, const float* pq,
                         const float* plc, int T1, int parts, int pstride, const int32_t* cand,
                         int V, int rule, float ratio, float delta, int32_t* tokens_out,
                         int32_t* n_accepted, int32_t* accept_out, int32_t* argmax_out,
                         float* pcand_out, float* entropy_out, hipStream_t s);

void launch_pack(const uint16_t* src, long R, int K, uint16_t* dst, hipStream_t s);
void launch_pack_pair(const uint16_t* gate, const uint16_t* up, long R, int K, uint16_t* dst,
                      hipStream_t s);

void launch_rmsnorm(const uint16_t* x, const float* gamma, float eps, int T, int H,
                    uint16_t* out, hipStream_t s);

// Violation words of the debug build, one per source file (see chk in
// device.hpp): each ORs its word into *out and clears it; 0 on success.
int debug_words_router(unsigned int* out);
int debug_words_experts(unsigned int* out);
int debug_words_head(unsigned int* out);
int debug_words_embed(unsigned int* out);

}  // namespace bdm
