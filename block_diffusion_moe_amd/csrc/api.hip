// extern "C" entry points of libbdmoe: argument validation, workspace
// carve-up and the launch sequence.  Declarations and contracts are in
// include/bdmoe.h.  Nothing here allocates memory or synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "bdmoe.h"
#include "internal.hpp"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the gate/up pair layout: up follows gate by one 16-row group
bool pair_ok(const uint16_t* gate, const uint16_t* up, int H) {
  return up == gate + static_cast<size_t>(16) * H;
}

int check_moe_shape(int T, int H, int I, int E, int k, int has_shared) {
  if (T < 1 || H < 1 || I < 1 || E < 1 || k < 1 || k > E) return BDM_ERR_INVALID_ARG;
  if (has_shared != 0 && has_shared != 1) return BDM_ERR_INVALID_ARG;
  if (T > BDM_MAX_TOKENS || H > BDM_MAX_HIDDEN || H % 64 != 0 || I > BDM_MAX_INTER ||
      I % 32 != 0 || E > BDM_MAX_EXPERTS || k > BDM_MAX_TOPK)
    return BDM_ERR_UNSUPPORTED_SHAPE;
  return BDM_OK;
}

// Workspace layout of the MoE layer.  Returns total bytes; fills `m` when
// `base` is given.
size_t moe_layout(int T, int H, int I, int E, int k, int has_shared, char* base,
                  bdm::MoeMeta* m) {
  const size_t P = static_cast<size_t>(T) * (k + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return base ? base + o : nullptr;
  };
  char* logits = take(sizeof(float) * bdm::kRouterParts * T * E);
  char* topk_idx = take(sizeof(int32_t) * T * k);
  char* topk_w = take(sizeof(float) * T * k);
  char* topk_p = take(sizeof(float) * T * k);
  char* cand_id = take(sizeof(int32_t) * T * bdm::kCoreCand);
  char* cand_l = take(sizeof(float) * T * bdm::kCoreCand);
  char* info = take(sizeof(int32_t) * 4);
  char* slots = take(sizeof(int) * 4 * bdm::moe_max_slots(T, E, k, has_shared));
  char* pair_rows = take(sizeof(int32_t) * P);
  char* act = take(sizeof(uint16_t) * P * I);
  char* ypair = take(sizeof(float) * P * H);
  if (m) {
    m->logits = reinterpret_cast<float*>(logits);
    m->topk_idx = reinterpret_cast<int32_t*>(topk_idx);
    m->topk_w = reinterpret_cast<float*>(topk_w);
    m->topk_p = reinterpret_cast<float*>(topk_p);
    m->cand_id = reinterpret_cast<int32_t*>(cand_id);
    m->cand_l = reinterpret_cast<float*>(cand_l);
    m->info = reinterpret_cast<int32_t*>(info);
    m->slots = reinterpret_cast<int4*>(slots);
    m->pair_rows = reinterpret_cast<int32_t*>(pair_rows);
    m->act = reinterpret_cast<uint16_t*>(act);
    m->ypair = reinterpret_cast<float*>(ypair);
  }
  return off;
}

int check_head_shape(int T, int H, int V) {
  if (T < 1 || H < 1 || V < 2) return BDM_ERR_INVALID_ARG;
  if (T > BDM_MAX_TOKENS || H > BDM_MAX_HIDDEN || H % 64 != 0) return BDM_ERR_UNSUPPORTED_SHAPE;
  return BDM_OK;
}

constexpr int kHeadMaxGrid = 1024;   // partials per token are sized for this many workgroups

size_t head_layout(int T, char* base, bdm::HeadParts* p) {
  const size_t n = static_cast<size_t>(T) * kHeadMaxGrid;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return base ? base + o : nullptr;
  };
  char* m = take(sizeof(float) * n);
  char* s = take(sizeof(float) * n);
  char* a = take(sizeof(int32_t) * n);
  if (p) {
    p->m = reinterpret_cast<float*>(m);
    p->s = reinterpret_cast<float*>(s);
    p->a = reinterpret_cast<int32_t*>(a);
  }
  return off;
}

// Verify epilogue partials: (m, s, a) as the head's plus q and lc.
struct VerifyParts {
  float* m;
  float* s;
  int32_t* a;
  float* q;
  float* lc;
};

size_t verify_layout(int T1, char* base, VerifyParts* p) {
  const size_t n = static_cast<size_t>(T1) * kHeadMaxGrid;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return base ? base + o : nullptr;
  };
  char* m = take(sizeof(float) * n);
  char* s = take(sizeof(float) * n);
  char* a = take(sizeof(int32_t) * n);
  char* q = take(sizeof(float) * n);
  char* lc = take(sizeof(float) * n);
  if (p) {
    p->m = reinterpret_cast<float*>(m);
    p->s = reinterpret_cast<float*>(s);
    p->a = reinterpret_cast<int32_t*>(a);
    p->q = reinterpret_cast<float*>(q);
    p->lc = reinterpret_cast<float*>(lc);
  }
  return off;
}

int check_verify_shape(int T1, int H, int V) {
  if (T1 < 1 || H < 1 || V < 2) return BDM_ERR_INVALID_ARG;
  if (T1 > BDM_MAX_TOKENS || H % 64 != 0) return BDM_ERR_UNSUPPORTED_SHAPE;
  const int ks = H / 256;
  if (H % 256 != 0 || (ks != 1 && ks != 2 && ks != 4 && ks != 8)) return BDM_ERR_UNSUPPORTED_SHAPE;
  return BDM_OK;
}

// The workspace of bdm_moe_block_forward_noalloc: a file-scope device array,
// one copy per device for the life of the process.  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address is
// taken once per device (hipGetSymbolAddress, with that device current, at
// the device's set-up below) and only that address is used.
static __device__ __align__(256) unsigned char scratch[BDM_STATIC_SCRATCH_BYTES];

// Per-device cache: compute-unit count, the device address of `scratch` and
// one-time kernel set-up.  Filled on the first call made with that device
// current; -1 marks a failed set-up.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<void*> g_scratch[kMaxDevices];

int device_setup(int* cus, void** scratch_ptr = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BDM_ERR_HIP;
  int n = g_cu_count[dev].load(std::memory_order_acquire);
  if (n == 0) {
    int v = 0;
    void* sp = nullptr;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0 || bdm::head_prepare() != 0 ||
        hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || sp == nullptr ||
        (reinterpret_cast<uintptr_t>(sp) % kAlign) != 0)
      v = -1;
    g_scratch[dev].store(sp, std::memory_order_relaxed);
    g_cu_count[dev].store(v, std::memory_order_release);
    n = v;
  }
  if (n < 0) return BDM_ERR_HIP;
  *cus = n;
  if (scratch_ptr) *scratch_ptr = g_scratch[dev].load(std::memory_order_relaxed);
  return BDM_OK;
}

int last_hip_status() {
  return hipGetLastError() == hipSuccess ? BDM_OK : BDM_ERR_HIP;
}

}  // namespace

extern "C" {

int bdm_version(void) { return 102; }

const char* bdm_status_string(int status) {
  switch (status) {
    case BDM_OK: return "ok";
    case BDM_ERR_INVALID_ARG: return "invalid argument";
    case BDM_ERR_UNSUPPORTED_SHAPE: return "shape outside the supported limits";
    case BDM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case BDM_ERR_HIP: return "HIP launch or runtime error";
    case BDM_ERR_NOT_DEBUG_BUILD: return "not the bounds-checked debug build";
    default: return "unknown status";
  }
}

int bdm_debug_bounds(unsigned int* violations) {
  if (!violations) return BDM_ERR_INVALID_ARG;
  *violations = 0u;
  if (!BDM_DEBUG_BOUNDS) return BDM_ERR_NOT_DEBUG_BUILD;
  if (hipDeviceSynchronize() != hipSuccess) return BDM_ERR_HIP;
  unsigned int w = 0u;
  if (bdm::debug_words_router(&w) || bdm::debug_words_experts(&w) ||
      bdm::debug_words_head(&w) || bdm::debug_words_embed(&w))
    return BDM_ERR_HIP;
  *violations = w;
  return BDM_OK;
}

int bdm_moe_workspace_bytes(int T, int H, int I, int E, int k, int has_shared, size_t* bytes) {
  if (!bytes) return BDM_ERR_INVALID_ARG;
  const int st = check_moe_shape(T, H, I, E, k, has_shared);
  if (st != BDM_OK) return st;
  *bytes = moe_layout(T, H, I, E, k, has_shared, nullptr, nullptr);
  return BDM_OK;
}

namespace {

int moe_forward(const uint16_t* x, int T, int H, const float* w_router, const float* router_bias,
                int E, int k, int renorm, float top_p, int block, const uint16_t* w_gate,
                const uint16_t* w_up, const uint16_t* w_down, int I, const uint16_t* ws_gate,
                const uint16_t* ws_up, const uint16_t* ws_down, int weight_layout,
                const uint16_t* residual, uint16_t* y, uint16_t* y_norm, uint16_t* x_norm,
                int32_t* topk_idx, float* topk_w, int32_t* n_kept, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !workspace)
    return BDM_ERR_INVALID_ARG;
  const int nshared = (ws_gate != nullptr) + (ws_up != nullptr) + (ws_down != nullptr);
  if (nshared != 0 && nshared != 3) return BDM_ERR_INVALID_ARG;
  if (renorm != 0 && renorm != 1) return BDM_ERR_INVALID_ARG;
  if (weight_layout != BDM_LAYOUT_ROW_MAJOR && weight_layout != BDM_LAYOUT_MFMA_TILES &&
      weight_layout != BDM_LAYOUT_MFMA_TILES_GU)
    return BDM_ERR_INVALID_ARG;
  const int has_shared = nshared == 3 ? 1 : 0;
  if (weight_layout == BDM_LAYOUT_MFMA_TILES_GU &&
      (!pair_ok(w_gate, w_up, H) || (has_shared && !pair_ok(ws_gate, ws_up, H))))
    return BDM_ERR_INVALID_ARG;
  int st = check_moe_shape(T, H, I, E, k, has_shared);
  if (st != BDM_OK) return st;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(y) || (residual && !aligned16(residual)) ||
      (y_norm && !aligned16(y_norm)) ||
      (has_shared && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(ws_down))) ||
      (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return BDM_ERR_INVALID_ARG;
  // x may be y only when the layer normalises x itself (the router reads x
  // before the combine writes y)
  if (static_cast<const void*>(x) == static_cast<const void*>(y) && !x_norm)
    return BDM_ERR_INVALID_ARG;
  if (y_norm && (static_cast<const void*>(y_norm) == static_cast<const void*>(y) ||
                 static_cast<const void*>(y_norm) == static_cast<const void*>(x) ||
                 static_cast<const void*>(y_norm) == static_cast<const void*>(residual)))
    return BDM_ERR_INVALID_ARG;
  if (x_norm && (!aligned16(x_norm) || static_cast<void*>(x_norm) == static_cast<const void*>(x) ||
                 static_cast<void*>(x_norm) == static_cast<void*>(y) ||
                 static_cast<void*>(x_norm) == static_cast<void*>(y_norm) ||
                 static_cast<const void*>(x_norm) == static_cast<const void*>(residual)))
    return BDM_ERR_INVALID_ARG;
  const size_t need = moe_layout(T, H, I, E, k, has_shared, nullptr, nullptr);
  if (workspace_bytes < need) return BDM_ERR_WORKSPACE_TOO_SMALL;

  int cus = 0;
  st = device_setup(&cus);
  if (st != BDM_OK) return st;
  bdm::MoeMeta meta;
  moe_layout(T, H, I, E, k, has_shared, static_cast<char*>(workspace), &meta);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // with x_norm the router normalises x and the experts read the result
  bdm::launch_router(x, T, H, w_router, router_bias, E, k, renorm, has_shared, top_p, block,
                     meta, topk_idx, topk_w, n_kept, x_norm, s);
  bdm::launch_experts(x_norm ? x_norm : x, T, H, I, E, k, has_shared, w_gate, w_up, w_down,
                      ws_gate, ws_up, ws_down, residual, y, y_norm, meta, weight_layout, s);
  return last_hip_status();
}

}  // namespace

int bdm_moe_block_forward(const uint16_t* x, int T, int H, const float* w_router,
                          const float* router_bias, int E, int k, int renorm,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          int I, const uint16_t* ws_gate, const uint16_t* ws_up,
                          const uint16_t* ws_down, int weight_layout, const uint16_t* residual,
                          uint16_t* y, uint16_t* y_norm, uint16_t* x_norm, int32_t* topk_idx,
                          float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward(x, T, H, w_router, router_bias, E, k, renorm, 0.0f, 0, w_gate, w_up, w_down,
                     I, ws_gate, ws_up, ws_down, weight_layout, residual, y, y_norm, x_norm,
                     topk_idx, topk_w, nullptr, workspace, workspace_bytes, stream);
}

int bdm_moe_block_forward_noalloc(const uint16_t* x, int T, int H, const float* w_router,
                                  const float* router_bias, int E, int k, int renorm,
                                  const uint16_t* w_gate, const uint16_t* w_up,
                                  const uint16_t* w_down, int I, const uint16_t* ws_gate,
                                  const uint16_t* ws_up, const uint16_t* ws_down,
                                  int weight_layout, const uint16_t* residual, uint16_t* y,
                                  uint16_t* y_norm, int32_t* topk_idx, float* topk_w,
                                  void* stream) {
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y) return BDM_ERR_INVALID_ARG;
  const int has_shared = (ws_gate != nullptr || ws_up != nullptr || ws_down != nullptr) ? 1 : 0;
  const int st = check_moe_shape(T, H, I, E, k, has_shared);
  if (st != BDM_OK) return st;
  // sizes whose workspace exceeds the static buffer: rejected before any
  // device call
  if (moe_layout(T, H, I, E, k, has_shared, nullptr, nullptr) > BDM_STATIC_SCRATCH_BYTES)
    return BDM_ERR_WORKSPACE_TOO_SMALL;
  int cus = 0;
  void* sp = nullptr;
  const int ds = device_setup(&cus, &sp);
  if (ds != BDM_OK) return ds;
  return moe_forward(x, T, H, w_router, router_bias, E, k, renorm, 0.0f, 0, w_gate, w_up, w_down,
                     I, ws_gate, ws_up, ws_down, weight_layout, residual, y, y_norm, nullptr,
                     topk_idx, topk_w, nullptr, sp, BDM_STATIC_SCRATCH_BYTES, stream);
}

int bdm_moe_block_forward_coreset(const uint16_t* x, int T, int H, const float* w_router,
                                  const float* router_bias, int E, int k, int renorm,
                                  float top_p, int block_tokens, const uint16_t* w_gate,
                                  const uint16_t* w_up, const uint16_t* w_down, int I,
                                  const uint16_t* ws_gate, const uint16_t* ws_up,
                                  const uint16_t* ws_down, int weight_layout,
                                  const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                                  uint16_t* x_norm, int32_t* topk_idx, float* topk_w,
                                  int32_t* n_kept, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return BDM_ERR_INVALID_ARG;
  if (block_tokens < 1 || block_tokens > BDM_CORESET_MAX_BLOCK) return BDM_ERR_INVALID_ARG;
  return moe_forward(x, T, H, w_router, router_bias, E, k, renorm, top_p, block_tokens, w_gate,
                     w_up, w_down, I, ws_gate, ws_up, ws_down, weight_layout, residual, y, y_norm,
                     x_norm, topk_idx, topk_w, n_kept, workspace, workspace_bytes, stream);
}

int bdm_head_workspace_bytes(int T, int H, int V, size_t* bytes) {
  if (!bytes) return BDM_ERR_INVALID_ARG;
  const int st = check_head_shape(T, H, V);
  if (st != BDM_OK) return st;
  *bytes = head_layout(T, nullptr, nullptr);
  return BDM_OK;
}

int bdm_lm_head_unmask(const uint16_t* h, int T, int H, const uint16_t* w_head, int V,
                       int weight_layout, int32_t mask_id, float threshold, int fallback,
                       int block_tokens, int32_t* tokens, int32_t* argmax, float* conf,
                       int32_t* n_committed, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!h || !w_head || !tokens || !workspace) return BDM_ERR_INVALID_ARG;
  int st = check_head_shape(T, H, V);
  if (st != BDM_OK) return st;
  if (mask_id < 0 || mask_id >= V) return BDM_ERR_INVALID_ARG;
  if (!(threshold == threshold) || threshold == INFINITY || threshold == -INFINITY)
    return BDM_ERR_INVALID_ARG;
  if (fallback != 0 && fallback != 1) return BDM_ERR_INVALID_ARG;
  if (block_tokens < 0) return BDM_ERR_INVALID_ARG;
  if (weight_layout != BDM_LAYOUT_ROW_MAJOR && weight_layout != BDM_LAYOUT_MFMA_TILES)
    return BDM_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_head) || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return BDM_ERR_INVALID_ARG;
  const size_t need = head_layout(T, nullptr, nullptr);
  if (workspace_bytes < need) return BDM_ERR_WORKSPACE_TOO_SMALL;
  int cus = 0;
  st = device_setup(&cus);
  if (st != BDM_OK) return st;
  bdm::HeadParts parts;
  head_layout(T, static_cast<char*>(workspace), &parts);
  parts.grid = cus < kHeadMaxGrid ? cus : kHeadMaxGrid;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  bdm::launch_head_stats(h, T, H, w_head, V, 0, weight_layout, mask_id, parts.m, parts.s, parts.a,
                         parts.grid, parts.grid, s);
  bdm::launch_unmask(parts.m, parts.s, parts.a, T, parts.grid, parts.grid, mask_id, threshold,
                     fallback, block_tokens, tokens, argmax, conf, n_committed, nullptr, s);
  return last_hip_status();
}

int bdm_head_verify_workspace_bytes(int T1, int H, int V, size_t* bytes) {
  if (!bytes) return BDM_ERR_INVALID_ARG;
  const int st = check_verify_shape(T1, H, V);
  if (st != BDM_OK) return st;
  *bytes = verify_layout(T1, nullptr, nullptr);
  return BDM_OK;
}

int bdm_lm_head_verify(const uint16_t* h, int T1, int H, const uint16_t* w_head, int V,
                       int weight_layout, const int32_t* cand, int rule, float ratio, float delta,
                       int32_t* tokens_out, int32_t* n_accepted, int32_t* accept, int32_t* argmax,
                       float* p_cand, float* entropy, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!h || !w_head || !tokens_out || !n_accepted || !workspace) return BDM_ERR_INVALID_ARG;
  if (T1 > 1 && !cand) return BDM_ERR_INVALID_ARG;
  int st = check_verify_shape(T1, H, V);
  if (st != BDM_OK) return st;
  if (rule != BDM_VERIFY_EXACT && rule != BDM_VERIFY_THRESHOLD) return BDM_ERR_INVALID_ARG;
  if (!(ratio == ratio) || !(delta == delta) || ratio == INFINITY || delta == INFINITY ||
      ratio == -INFINITY || delta == -INFINITY)
    return BDM_ERR_INVALID_ARG;
  if (weight_layout != BDM_LAYOUT_ROW_MAJOR && weight_layout != BDM_LAYOUT_MFMA_TILES)
    return BDM_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_head) || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return BDM_ERR_INVALID_ARG;
  const size_t need = verify_layout(T1, nullptr, nullptr);
  if (workspace_bytes < need) return BDM_ERR_WORKSPACE_TOO_SMALL;
  int cus = 0;
  st = device_setup(&cus);
  if (st != BDM_OK) return st;
  VerifyParts p;
  verify_layout(T1, static_cast<char*>(workspace), &p);
  const int grid = cus < kHeadMaxGrid ? cus : kHeadMaxGrid;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  bdm::launch_head_verify_stats(h, T1, H, w_head, V, weight_layout, cand, T1 - 1, p.m, p.s, p.a,
                                p.q, p.lc, grid, grid, s);
  bdm::launch_verify_merge(p.m, p.s, p.a, p.q, p.lc, T1, grid, grid, cand, V, rule, ratio, delta,
                           tokens_out, n_accepted, accept, argmax, p_cand, entropy, s);
  return last_hip_status();
}

int bdm_head_stat_parts(int* parts) {
  if (!parts) return BDM_ERR_INVALID_ARG;
  int cus = 0;
  const int st = device_setup(&cus);
  if (st != BDM_OK) return st;
  *parts = cus < kHeadMaxGrid ? cus : kHeadMaxGrid;
  return BDM_OK;
}

int bdm_lm_head_stats(const uint16_t* h, int T, int H, const uint16_t* w_head, int V,
                      int vocab_offset, int weight_layout, int32_t mask_id, float* stat_max,
                      float* stat_sum, int32_t* stat_arg, int stat_stride, void* stream) {
  if (!h || !w_head || !stat_max || !stat_sum || !stat_arg) return BDM_ERR_INVALID_ARG;
  int st = check_head_shape(T, H, V < 2 ? 2 : V);
  if (st != BDM_OK) return st;
  if (V < 1 || vocab_offset < 0 || vocab_offset > 0x7fffffff - V) return BDM_ERR_INVALID_ARG;
  if (weight_layout != BDM_LAYOUT_ROW_MAJOR && weight_layout != BDM_LAYOUT_MFMA_TILES)
    return BDM_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_head)) return BDM_ERR_INVALID_ARG;
  int parts = 0;
  st = bdm_head_stat_parts(&parts);
  if (st != BDM_OK) return st;
  if (stat_stride < parts) return BDM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  bdm::launch_head_stats(h, T, H, w_head, V, vocab_offset, weight_layout, mask_id, stat_max,
                         stat_sum, stat_arg, stat_stride, parts, static_cast<hipStream_t>(stream));
  return last_hip_status();
}

int bdm_unmask_from_stats(const float* stat_max, const float* stat_sum, const int32_t* stat_arg,
                          int T, int parts, int stat_stride, int32_t mask_id, float threshold,
                          int fallback, int block_tokens, int32_t* tokens, int32_t* argmax,
                          float* conf, int32_t* n_committed, void* stream) {
  if (!stat_max || !stat_sum || !stat_arg || !tokens) return BDM_ERR_INVALID_ARG;
  if (T < 1 || parts < 1 || stat_stride < parts) return BDM_ERR_INVALID_ARG;
  if (T > BDM_MAX_TOKENS) return BDM_ERR_UNSUPPORTED_SHAPE;
  if (!(threshold == threshold) || threshold == INFINITY || threshold == -INFINITY)
    return BDM_ERR_INVALID_ARG;
  if (fallback != 0 && fallback != 1) return BDM_ERR_INVALID_ARG;
  if (block_tokens < 0) return BDM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  bdm::launch_unmask(stat_max, stat_sum, stat_arg, T, parts, stat_stride, mask_id, threshold,
                     fallback, block_tokens, tokens, argmax, conf, n_committed, nullptr,
                     static_cast<hipStream_t>(stream));
  return last_hip_status();
}

// Workspace of the denoise loop: the MoE layer's, the head's partials, the
// block's hidden state and its normalised copy, two step counters.
size_t denoise_layout(int T, int H, int I, int E, int k, int has_shared, char* base,
                      bdm::MoeMeta* meta, bdm::HeadParts* parts, uint16_t** x, uint16_t** xn,
                      int32_t** counters) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return base ? base + o : nullptr;
  };
  const size_t nm = moe_layout(T, H, I, E, k, has_shared, nullptr, nullptr);
  char* m = take(nm);
  const size_t nh = head_layout(T, nullptr, nullptr);
  char* h = take(nh);
  char* xa = take(sizeof(uint16_t) * static_cast<size_t>(T) * H);
  char* xb = take(sizeof(uint16_t) * static_cast<size_t>(T) * H);
  char* c = take(sizeof(int32_t) * 4);
  if (base) {
    moe_layout(T, H, I, E, k, has_shared, m, meta);
    head_layout(T, h, parts);
    *x = reinterpret_cast<uint16_t*>(xa);
    *xn = reinterpret_cast<uint16_t*>(xb);
    *counters = reinterpret_cast<int32_t*>(c);
  }
  return off;
}

int bdm_denoise_workspace_bytes(int T, int H, int I, int E, int k, int has_shared,
                                size_t* bytes) {
  if (!bytes) return BDM_ERR_INVALID_ARG;
  const int st = check_moe_shape(T, H, I, E, k, has_shared);
  if (st != BDM_OK) return st;
  *bytes = denoise_layout(T, H, I, E, k, has_shared, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr);
  return BDM_OK;
}

int bdm_denoise_block(int32_t* tokens, int T, const uint16_t* w_embed, int V, int H,
                      const bdm_moe_layer* layers, int L, int E, int k, int I, int renorm,
                      const uint16_t* w_head, int weight_layout, int32_t mask_id, float threshold,
                      float coreset_top_p, int block_tokens, int max_steps, int* steps_taken,
                      int32_t* commits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!tokens || !w_embed || !w_head || !steps_taken || !workspace || (L > 0 && !layers))
    return BDM_ERR_INVALID_ARG;
  if (L < 0 || max_steps < 0 || (renorm != 0 && renorm != 1)) return BDM_ERR_INVALID_ARG;
  if (weight_layout != BDM_LAYOUT_ROW_MAJOR && weight_layout != BDM_LAYOUT_MFMA_TILES &&
      weight_layout != BDM_LAYOUT_MFMA_TILES_GU)
    return BDM_ERR_INVALID_ARG;
  // the head is packed plainly when the experts use the gate/up pair layout
  const int head_layout_ =
      weight_layout == BDM_LAYOUT_MFMA_TILES_GU ? BDM_LAYOUT_MFMA_TILES : weight_layout;
  if (!(threshold == threshold) || threshold == INFINITY || threshold == -INFINITY)
    return BDM_ERR_INVALID_ARG;
  if (!(coreset_top_p >= 0.0f && coreset_top_p <= 1.0f)) return BDM_ERR_INVALID_ARG;
  if (block_tokens < 0) return BDM_ERR_INVALID_ARG;
  // the rule's blocks (0: the whole call) and the coreset selector's
  const int B = (block_tokens == 0 || block_tokens > T) ? T : block_tokens;
  const int cs_block = B < BDM_CORESET_MAX_BLOCK ? B : BDM_CORESET_MAX_BLOCK;
  int has_shared = 1;
  for (int l = 0; l < L; ++l) {
    const bdm_moe_layer& w = layers[l];
    if (!w.w_router || !w.w_gate || !w.w_up || !w.w_down) return BDM_ERR_INVALID_ARG;
    const int ns = (w.ws_gate != nullptr) + (w.ws_up != nullptr) + (w.ws_down != nullptr);
    if (ns != 0 && ns != 3) return BDM_ERR_INVALID_ARG;
    if (l == 0) has_shared = ns == 3;
    else if ((ns == 3) != (has_shared == 1)) return BDM_ERR_INVALID_ARG;
    if (!aligned16(w.w_router) || !aligned16(w.w_gate) || !aligned16(w.w_up) ||
        !aligned16(w.w_down) ||
        (ns == 3 && (!aligned16(w.ws_gate) || !aligned16(w.ws_up) || !aligned16(w.ws_down))))
      return BDM_ERR_INVALID_ARG;
    if (weight_layout == BDM_LAYOUT_MFMA_TILES_GU &&
        (!pair_ok(w.w_gate, w.w_up, H) || (ns == 3 && !pair_ok(w.ws_gate, w.ws_up, H))))
      return BDM_ERR_INVALID_ARG;
  }
  int st = check_moe_shape(T, H, I, E, k, has_shared);
  if (st != BDM_OK) return st;
  st = check_head_shape(T, H, V);
  if (st != BDM_OK) return st;
  if (mask_id < 0 || mask_id >= V) return BDM_ERR_INVALID_ARG;
  if (!aligned16(w_embed) || !aligned16(w_head) ||
      (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return BDM_ERR_INVALID_ARG;
  const size_t need = denoise_layout(T, H, I, E, k, has_shared, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr);
  if (workspace_bytes < need) return BDM_ERR_WORKSPACE_TOO_SMALL;
  int cus = 0;
  st = device_setup(&cus);
  if (st != BDM_OK) return st;

  bdm::MoeMeta meta;
  bdm::HeadParts parts;
  uint16_t *x = nullptr, *xn = nullptr;
  int32_t* cnt = nullptr;
  denoise_layout(T, H, I, E, k, has_shared, static_cast<char*>(workspace), &meta, &parts, &x, &xn,
                 &cnt);
  parts.grid = cus < kHeadMaxGrid ? cus : kHeadMaxGrid;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int steps = 0;
  *steps_taken = 0;
  while (steps < max_steps) {
    bdm::launch_embed(tokens, T, w_embed, V, H, x, xn, s);     // x and RMSNorm(x)
    // each layer's combine also writes RMSNorm of its output: the next
    // layer's input, after the last layer the final norm
    for (int l = 0; l < L; ++l) {
      const bdm_moe_layer& w = layers[l];
      bdm::launch_router(xn, T, H, w.w_router, w.router_bias, E, k, renorm, has_shared,
                         coreset_top_p, cs_block, meta, nullptr, nullptr, nullptr, nullptr, s);
      bdm::launch_experts(xn, T, H, I, E, k, has_shared, w.w_gate, w.w_up, w.w_down, w.ws_gate,
                          w.ws_up, w.ws_down, x, x, xn, meta, weight_layout, s);
    }
    bdm::launch_head_stats(xn, T, H, w_head, V, 0, head_layout_, mask_id, parts.m, parts.s,
                           parts.a, parts.grid, parts.grid, s);
    bdm::launch_unmask(parts.m, parts.s, parts.a, T, parts.grid, parts.grid, mask_id, threshold,
                       1, B, tokens, nullptr, nullptr, cnt, cnt + 1, s);
    int32_t host[2] = {0, 0};
    if (hipMemcpyAsync(host, cnt, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return BDM_ERR_HIP;
    st = last_hip_status();
    if (st != BDM_OK) return st;
    if (commits) commits[steps] = host[0];
    ++steps;
    *steps_taken = steps;
    if (host[1] <= 0 || host[0] <= 0) break;      // nothing masked is left
  }
  return BDM_OK;
}

int bdm_packed_weight_elems(long rows, int cols, size_t* n) {
  if (!n || rows < 1 || cols < 32 || cols % 32 != 0) return BDM_ERR_INVALID_ARG;
  *n = static_cast<size_t>((rows + 15) / 16) * 16 * static_cast<size_t>(cols);
  return BDM_OK;
}

int bdm_pack_weights(const uint16_t* src, long rows, int cols, uint16_t* dst, void* stream) {
  size_t n = 0;
  const int st = bdm_packed_weight_elems(rows, cols, &n);
  if (st != BDM_OK) return st;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return BDM_ERR_INVALID_ARG;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), a1 = a0 + 2 * static_cast<size_t>(rows) * cols;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(dst), b1 = b0 + 2 * n;
  if (a0 < b1 && b0 < a1) return BDM_ERR_INVALID_ARG;          // overlap
  if ((rows + 15) / 16 * (cols / 32) > 4L * 0x7fffffffL) return BDM_ERR_UNSUPPORTED_SHAPE;
  (void)hipGetLastError();
  bdm::launch_pack(src, rows, cols, dst, static_cast<hipStream_t>(stream));
  return last_hip_status();
}

int bdm_pack_gate_up(const uint16_t* gate, const uint16_t* up, long rows, int cols,
                     uint16_t* dst, void* stream) {
  if (!gate || !up || !dst || rows < 16 || rows % 16 != 0 || cols < 32 || cols % 32 != 0)
    return BDM_ERR_INVALID_ARG;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(dst)) return BDM_ERR_INVALID_ARG;
  if ((rows / 16) * (cols / 32) > 4L * 0x7fffffffL) return BDM_ERR_UNSUPPORTED_SHAPE;
  const size_t n = static_cast<size_t>(rows) * cols;        // elements of one matrix
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), d1 = d0 + 2 * n * sizeof(uint16_t);
  auto overlaps = [&](const uint16_t* src) {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), s1 = s0 + n * sizeof(uint16_t);
    return s0 < d1 && d0 < s1;
  };
  if (overlaps(gate) || overlaps(up)) return BDM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  bdm::launch_pack_pair(gate, up, rows, cols, dst, static_cast<hipStream_t>(stream));
  return last_hip_status();
}

int bdm_rmsnorm(const uint16_t* x, const float* gamma, float eps, int T, int H, uint16_t* out,
                void* stream) {
  if (!x || !out || T < 1 || H < 1) return BDM_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps == INFINITY) return BDM_ERR_INVALID_ARG;
  if (H % 64 != 0 || H > BDM_MAX_HIDDEN) return BDM_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return BDM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  bdm::launch_rmsnorm(x, gamma, eps, T, H, out, static_cast<hipStream_t>(stream));
  return last_hip_status();
}

}  // extern "C"
