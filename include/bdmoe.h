/*
 * bdmoe.h -- C ABI of the block-diffusion MoE denoise-step library (libbdmoe.so)
 *
 * One denoising step of a block-diffusion mixture-of-experts language model
 * shaped like Clover-35B-A3B, on one AMD Instinct MI355X (gfx950): the routed
 * MoE feed-forward layer applied to a whole block of positions at once, the
 * RMSNorm between layers, and the untied output head fused with the
 * low-confidence unmask rule.
 *
 * Pages cited (title, then section):
 *   [files]  "Clover-35B-A3B: how a diffusion model gets to 680 tokens a
 *            second, read from its files"
 *   [deep]   "Deep Dive -- Clover 35B: a diffusion LLM at Qwen parity, 680 tok/s"
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers (HBM of the current HIP device)
 *     unless stated otherwise.  bf16 tensors are passed as uint16_t bit
 *     patterns.  All tensors are dense row-major with the last dimension
 *     contiguous; no strides.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *     only enqueue kernels on it and return; they never synchronise.  Outputs
 *     are valid once the stream has reached the enqueued work.
 *   - Ownership: the caller owns every buffer, before, during and after the
 *     call.  The library allocates no device or host memory and keeps no state
 *     besides a per-device cache of device properties.
 *   - Workspace: device scratch of at least the size returned by the matching
 *     *_workspace_bytes query, 256-byte aligned.  Its contents on entry are
 *     ignored; on return it holds intermediate results (undefined to callers).
 *     Two calls that run concurrently need two workspaces.
 *   - Errors: 0 on success, otherwise a negative BDM_ERR_* code.  All argument
 *     checks run before anything is enqueued, so a failed check leaves every
 *     output untouched.  BDM_ERR_HIP means a launch failed after validation
 *     (outputs then undefined).  The library never aborts or prints.
 *   - Repeatability: identical inputs give bitwise-identical outputs (no
 *     floating-point atomics; every reduction has a fixed order).
 *   - Thread safety: calls on different streams may be issued from different
 *     host threads as long as their workspaces and outputs are distinct.
 */
#ifndef BDMOE_H
#define BDMOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define BDM_API __attribute__((visibility("default")))
#else
#define BDM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define BDM_OK                       0
#define BDM_ERR_INVALID_ARG         -1  /* null pointer, bad size, bad flag */
#define BDM_ERR_UNSUPPORTED_SHAPE   -2  /* legal sizes outside the kernels' limits */
#define BDM_ERR_WORKSPACE_TOO_SMALL -3
#define BDM_ERR_HIP                 -4  /* a HIP call failed */
#define BDM_ERR_NOT_DEBUG_BUILD     -5  /* bdm_debug_bounds on the release library */

/* [files] "What Clover is": mask_token_id 151669, low_confidence threshold 0.95 */
#define BDM_MASK_ID_CLOVER     151669
#define BDM_THRESHOLD_DEFAULT  0.95f

/* Layout of the bf16 weight matrices a call reads (argument weight_layout).
 *   BDM_LAYOUT_ROW_MAJOR     [rows][cols], cols contiguous (the natural layout)
 *   BDM_LAYOUT_MFMA_TILES    the packed layout bdm_pack_weights produces: 1 KB
 *                            tiles of 16 rows x 32 cols in MFMA operand order,
 *                            a 16-row group contiguous over all cols.  The
 *                            same values; only the byte order differs (streams
 *                            at a higher fraction of HBM bandwidth).
 *   BDM_LAYOUT_MFMA_TILES_GU MoE layer only: down (and the head) as in
 *                            BDM_LAYOUT_MFMA_TILES, gate and up (routed, and
 *                            the shared expert's) as one buffer written by
 *                            bdm_pack_gate_up, whose 16-row groups alternate
 *                            gate, up; then w_up = w_gate + 16*H elements
 *                            (ws_up = ws_gate + 16*H), checked.  A gate/up
 *                            work item then streams one contiguous run. */
#define BDM_LAYOUT_ROW_MAJOR     0
#define BDM_LAYOUT_MFMA_TILES    1
#define BDM_LAYOUT_MFMA_TILES_GU 2

/* Limits of this implementation (checked; BDM_ERR_UNSUPPORTED_SHAPE beyond). */
#define BDM_MAX_TOKENS   2048   /* T: positions per call (up to 64 blocks of 32 stacked) */
#define BDM_MAX_HIDDEN   2048   /* H, multiple of 64 */
#define BDM_MAX_INTER    1024   /* I, multiple of 32 */
#define BDM_MAX_EXPERTS  1024   /* E */
#define BDM_MAX_TOPK       16   /* k, 1 <= k <= E */
#define BDM_CORESET_MAX_BLOCK 32 /* tokens per block of the coreset selector */

/* Library version as 10000*major + 100*minor + patch. */
BDM_API int bdm_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
BDM_API const char* bdm_status_string(int status);

/*
 * bdm_debug_bounds -- the bounds checks of the debug build.
 *
 * The library is also built as libbdmoe_debug.so (BDM_DEBUG_BOUNDS=1), the
 * same entry points with a device-side check on every index the kernels
 * read from memory or derive from what they read: slot-table entries, pair
 * rows, expert picks, re-route candidates and ranks, token ids given to the
 * embedding gather, head row groups and partial indices.  A check that
 * fails sets one bit of a violation word (the bit numbers are the kChk*
 * codes of the kernels' device header: 0 slot entry, 1 pair row, 2 expert
 * id, 3 token row, 4 vocabulary row, 5 token id, 6 softmax partial, 7
 * re-route candidate or rank, 8 workspace table index) and the index is
 * clamped into its buffer, so the call still completes.
 *
 * Writes the OR of the words of every kernel file, on the current device,
 * to *violations and clears them.  It synchronises with the device's work
 * (call it after the calls it checks have been ordered before it).
 * Returns BDM_OK; BDM_ERR_NOT_DEBUG_BUILD from the release library (which
 * has no checks; *violations is set to 0); BDM_ERR_INVALID_ARG for a NULL
 * pointer; BDM_ERR_HIP if reading the words fails.
 */
BDM_API int bdm_debug_bounds(unsigned int* violations);

/*
 * bdm_moe_workspace_bytes -- workspace size for bdm_moe_block_forward.
 *   T, H, I, E, k, has_shared: as in bdm_moe_block_forward.
 *   bytes: HOST pointer that receives the size.
 * Returns BDM_OK, or the same validation error bdm_moe_block_forward would
 * return for these sizes.  Pure host arithmetic; needs no GPU.
 */
BDM_API int bdm_moe_workspace_bytes(int T, int H, int I, int E, int k, int has_shared, size_t* bytes);

/*
 * bdm_moe_block_forward -- one routed MoE feed-forward layer over a block.
 *
 * [files] "What Clover is": a layer holds 256 routed experts; each token is
 * sent to 8 of them, and a 257th, shared expert serves every token; gate and
 * up map 2,048 to 512 and down maps 512 back to 2,048.  [deep] "What
 * DiffuSpace actually shipped": the same top-8 plus shared-expert layout.
 * [files] "The expert selection": a block's step reads every expert that any
 * of its tokens picked, so the layer is computed per expert over all the
 * block's tokens routed to it.
 *
 * For every token t (row of x), independently:
 *   l      = fp32(x_t) . w_router^T (+ router_bias)             fp32 logits [E]
 *   S_t    = the k experts with the largest l (equal: lower id first),
 *            ordered by decreasing l
 *   w_t,j  = softmax(l)[S_j] / sum_{i in S} softmax(l)[i]   if renorm
 *          = softmax(l)[S_j]                                 otherwise
 *   Y_e(x) = W_down,e . bf16( silu(W_gate,e . x) * (W_up,e . x) ),
 *            silu(z) = z / (1 + e^-z), fp32 accumulation
 *   y_t    = bf16( residual_t + sum_{j<k} w_t,j Y_{S_j}(x_t) + Y_shared(x_t) )
 *            summed in fp32 in that order (residual 0 when NULL; the shared
 *            term only when the ws_* trio is given)
 *
 * Arguments
 *   x            [T][H] bf16        block activations (T tokens)
 *   w_router     [E][H] fp32        router weights
 *   router_bias  [E] fp32 or NULL   added to the logits before softmax/top-k
 *   E, k         experts, experts per token (1 <= k <= min(E, 16))
 *   renorm       1: renormalise the k weights to sum to 1; 0: raw softmax
 *   w_gate,w_up  [E][I][H] bf16     routed experts, output-major
 *   w_down       [E][H][I] bf16
 *   I            expert intermediate size (multiple of 32, <= 1024)
 *   ws_gate, ws_up [I][H], ws_down [H][I] bf16: the shared expert; all three
 *                NULL = no shared expert (mixing NULL and non-NULL is an error)
 *   weight_layout layout of w_gate, w_up, w_down and ws_*: BDM_LAYOUT_ROW_MAJOR,
 *                or BDM_LAYOUT_MFMA_TILES with w_gate/w_up packed as one
 *                [E*I][H] matrix, w_down as [E*H][I], ws_gate/ws_up as [I][H]
 *                and ws_down as [H][I], or BDM_LAYOUT_MFMA_TILES_GU with
 *                w_gate/w_up (and ws_gate/ws_up) from bdm_pack_gate_up and
 *                the down matrices as in BDM_LAYOUT_MFMA_TILES (the router
 *                stays fp32 row-major)
 *   residual     [T][H] bf16 or NULL; may be the same pointer as y
 *   y            [T][H] bf16        output
 *   y_norm       [T][H] bf16 or NULL: also receives RMSNorm(y) (eps 1e-6,
 *                unit gamma; bit for bit what bdm_rmsnorm gives on y), the
 *                next layer's input in a pre-norm stack; must not alias x, y
 *                or residual
 *   x_norm       [T][H] bf16 or NULL.  When given, x is the layer's
 *                un-normalised input: the layer itself takes RMSNorm(x)
 *                (eps 1e-6, unit gamma; bit for bit what bdm_rmsnorm gives),
 *                writes it here and routes and runs the experts on it, i.e.
 *                y = residual + MoE(RMSNorm(x)) without a separate RMSNorm
 *                call; x may then be y (and residual).  Must not alias x, y,
 *                y_norm or residual.
 *   topk_idx     [T][k] int32 or NULL   receives S_t (decreasing weight)
 *   topk_w       [T][k] fp32 or NULL    receives w_t
 *   workspace, workspace_bytes: see bdm_moe_workspace_bytes
 * Limits: T <= 2048, H multiple of 64 and <= 2048, E <= 1024.
 *   Pointers 16-byte aligned (workspace 256-byte aligned).  NaN inputs give
 *   undefined values, never an out-of-bounds access.
 * No other aliasing is allowed.
 * (The argument list grew x_norm in library version 101.)
 *
 * Several blocks in one call (multi-block batching): stack the blocks' rows
 * in x (T = 32 x blocks, up to 64 blocks).  Tokens never interact, so each
 * row of y, topk_idx and topk_w is bit for bit what a call with that row's
 * block alone gives; the call reads each touched expert's weights once per
 * 64 of its tokens instead of once per block.
 */
BDM_API int bdm_moe_block_forward(const uint16_t* x, int T, int H,
                          const float* w_router, const float* router_bias, int E, int k,
                          int renorm,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          int I,
                          const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                          int weight_layout,
                          const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                          uint16_t* x_norm, int32_t* topk_idx, float* topk_w,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * bdm_moe_block_forward_noalloc -- bdm_moe_block_forward without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * The same computation, kernels and bits as bdm_moe_block_forward with
 * x_norm = NULL (x is the normalised input); the
 * workspace is instead a static device buffer of BDM_STATIC_SCRATCH_BYTES
 * inside the library, one per device, held until the process ends (its
 * address is looked up once per device at the library's first call on that
 * device).  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Arguments as in bdm_moe_block_forward, without
 * x_norm, workspace and workspace_bytes.
 * Limits: sizes whose bdm_moe_workspace_bytes exceed BDM_STATIC_SCRATCH_BYTES
 * (e.g. T = 256 fits at the Clover shape, T = 2048 does not) return
 * BDM_ERR_WORKSPACE_TOO_SMALL before any device call.
 * Every call on a device uses that device's one buffer: two calls that may
 * overlap on one device (different streams, different host threads) race;
 * serialise them (e.g. one stream).  The buffer keeps the last call's
 * intermediate results; nothing in it needs to start at zero.
 */
#define BDM_STATIC_SCRATCH_BYTES (32u << 20)

BDM_API int bdm_moe_block_forward_noalloc(const uint16_t* x, int T, int H,
                          const float* w_router, const float* router_bias, int E, int k,
                          int renorm,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          int I,
                          const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                          int weight_layout,
                          const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                          int32_t* topk_idx, float* topk_w, void* stream);

/*
 * bdm_moe_block_forward_coreset -- the same layer with the block coreset
 * expert selector in front of the experts.
 *
 * [files] "The expert selection": for a block, every token's top-8 routing
 * probabilities are added up per expert, the experts are sorted by that
 * total, the smallest set whose share of the total reaches top_p is kept
 * (never fewer than the top expert), and no token of the block may route
 * outside it; [files] "What Clover is": the selector is on with top_p 0.9.
 *
 * For every block of block_tokens consecutive rows of x (the last one may be
 * shorter), with p_t = softmax(l_t) over all E and S_t the first-pass picks
 * of bdm_moe_block_forward:
 *   mass_e = sum over the block's tokens, in order, of p_t[e] for e in S_t
 *            (fp32)
 *   order  = experts with mass > 0, larger mass first (equal: lower id)
 *   kept   = the shortest prefix of order whose cumulative mass (fp32, in
 *            that order) reaches top_p * total mass; at least one expert
 *   S'_t   = the min(k, |kept|) kept experts with the largest l_t (equal:
 *            lower id); w'_t as in bdm_moe_block_forward with the logits of
 *            the other experts at -inf; slots past |S'_t| hold expert -1
 *            and weight 0 and contribute nothing
 * and then y as in bdm_moe_block_forward with S', w'.
 *
 * Arguments as in bdm_moe_block_forward, plus
 *   top_p         in (0, 1]; 1 keeps every touched expert
 *   block_tokens  tokens per block, 1 .. BDM_CORESET_MAX_BLOCK (32)
 *   n_kept        [ceil(T / block_tokens)] int32 device array or NULL:
 *                 receives |kept| per block
 *   topk_idx/topk_w receive S', w' (-1 / 0 in the empty slots)
 * Workspace: bdm_moe_workspace_bytes for the same sizes.  Errors as in
 * bdm_moe_block_forward; top_p or block_tokens out of range ->
 * BDM_ERR_INVALID_ARG.
 */
BDM_API int bdm_moe_block_forward_coreset(const uint16_t* x, int T, int H,
                          const float* w_router, const float* router_bias, int E, int k,
                          int renorm, float top_p, int block_tokens,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          int I,
                          const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                          int weight_layout,
                          const uint16_t* residual, uint16_t* y, uint16_t* y_norm,
                          uint16_t* x_norm, int32_t* topk_idx, float* topk_w, int32_t* n_kept,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * bdm_moe_layer -- the device weights of one MoE layer for bdm_denoise_block
 * (the arrays of bdm_moe_block_forward; router_bias and the ws_* trio may be
 * NULL, the trio all or none and the same choice in every layer).
 */
typedef struct bdm_moe_layer {
  const float* w_router;       /* [E][H] fp32 */
  const float* router_bias;    /* [E] fp32 or NULL */
  const uint16_t* w_gate;      /* [E][I][H] bf16 */
  const uint16_t* w_up;        /* [E][I][H] bf16 */
  const uint16_t* w_down;      /* [E][H][I] bf16 */
  const uint16_t* ws_gate;     /* [I][H] bf16 or NULL */
  const uint16_t* ws_up;       /* [I][H] bf16 or NULL */
  const uint16_t* ws_down;     /* [H][I] bf16 or NULL */
} bdm_moe_layer;

/*
 * bdm_denoise_workspace_bytes -- workspace size for bdm_denoise_block (host
 * arithmetic; same validation as bdm_moe_workspace_bytes).
 */
BDM_API int bdm_denoise_workspace_bytes(int T, int H, int I, int E, int k, int has_shared,
                                        size_t* bytes);

/*
 * bdm_denoise_block -- the denoise loop over one block.
 *
 * [files] "How it writes": every slot of a new block holds the mask token; a
 * step runs the model on all slots at once, predicts each slot (mask logit
 * excluded) with its probability, fills the masked slots that reach the
 * threshold (or, if none does, the most confident one), and steps repeat
 * until the block holds no mask; a filled slot is never rewritten.
 * The model here is the expert part of the stack only (pre-norm):
 *   x = w_embed[tokens];  for each layer: x = bf16(x + MoE(RMSNorm(x)));
 *   h = RMSNorm(x);  tokens = unmask(head(h))        (RMSNorm eps 1e-6, gamma 1)
 * with MoE = bdm_moe_block_forward, the head and rule = bdm_lm_head_unmask
 * with the fallback on.  With coreset_top_p > 0 every layer's MoE is
 * bdm_moe_block_forward_coreset ([files] "What Clover is": the selector
 * ships on at top_p 0.9).
 *
 * Arguments
 *   tokens      [T] int32 device, in/out: the block (mask_id = masked slot)
 *   w_embed     [V][H] bf16 device, row-major: embedding rows
 *   layers      HOST array of L bdm_moe_layer (device pointers inside)
 *   E, k, I, renorm   as in bdm_moe_block_forward, the same for every layer
 *   w_head      [V][H] bf16 device: the untied head
 *   weight_layout     layout of every expert matrix and of w_head
 *                     (BDM_LAYOUT_MFMA_TILES_GU: the experts as in
 *                     bdm_moe_block_forward, w_head packed plainly)
 *   mask_id, threshold   as in bdm_lm_head_unmask
 *   coreset_top_p  0: plain top-k routing; in (0, 1]: the block coreset
 *               expert selector at that top_p in every layer (over blocks
 *               of min(block, 32) tokens)
 *   block_tokens  several blocks in one call: the T rows are blocks of this
 *               many slots, each with its own commit rule (every step
 *               commits at least one slot of every block still masked); the
 *               loop runs until no block has a masked slot.  0: one block
 *   max_steps   steps at most (the loop also stops when no slot is masked)
 *   steps_taken HOST int: steps run
 *   commits     HOST [max_steps] int32 or NULL: slots committed per step
 *   workspace   bdm_denoise_workspace_bytes(T, H, I, E, k, has_shared)
 * Synchronous: after each step the host waits for the step on `stream` and
 * reads two counters.  Errors as in bdm_moe_block_forward and
 * bdm_lm_head_unmask; BDM_ERR_HIP if a step fails.
 */
BDM_API int bdm_denoise_block(int32_t* tokens, int T, const uint16_t* w_embed, int V, int H,
                              const bdm_moe_layer* layers, int L, int E, int k, int I,
                              int renorm, const uint16_t* w_head, int weight_layout,
                              int32_t mask_id, float threshold, float coreset_top_p,
                              int block_tokens, int max_steps, int* steps_taken,
                              int32_t* commits, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * bdm_head_workspace_bytes -- workspace size for bdm_lm_head_unmask.
 *   bytes: HOST pointer.  Pure host arithmetic.
 */
BDM_API int bdm_head_workspace_bytes(int T, int H, int V, size_t* bytes);

/*
 * bdm_lm_head_unmask -- untied output head fused with the unmask rule.
 *
 * [files] "What Clover is": the head has its own weights (not the
 * embedding's), 248,320 x 2,048 = 508,559,360 of them, and every step streams
 * all of them.  [files] "How it writes", steps 2-3: each slot's prediction is
 * its highest-scoring token other than the mask token, with that token's
 * probability as confidence; masked slots at or above the threshold are
 * filled, and when no slot qualifies the most confident masked slot is filled
 * alone.
 *
 *   l_t     = fp32 logits h_t . w_head^T for all V rows (never stored)
 *   l_t[mask_id] = -inf
 *   argmax_t = argmax_v l_t (equal logits: lowest id)
 *   conf_t   = max_v softmax(l_t) = 1 / sum_v exp(l_t,v - max l_t)
 *   rule: for every t with tokens[t] == mask_id: commit (tokens[t] =
 *         argmax_t) iff conf_t >= threshold.  If fallback != 0 and no row
 *         committed but some row is masked, commit the masked row with the
 *         largest conf_t (equal: lowest t).  Other rows are never changed.
 *   A row with no finite logit (all -inf or NaN, e.g. a NaN hidden row) or
 *   whose sum of exponentials is NaN has no prediction: argmax_t = -1,
 *   conf_t = 0, and the rule never commits it (nor picks it as the
 *   fallback); it stays masked and n_committed does not count it.
 *
 * Arguments
 *   h            [T][H] bf16        final hidden states of the block
 *   w_head       [V][H] bf16        output head, vocabulary-row-major, or
 *                                  packed (weight_layout = BDM_LAYOUT_MFMA_TILES)
 *   mask_id      0 <= mask_id < V   (V >= 2)
 *   threshold    commit threshold (finite, compared with >=)
 *   fallback     1: the progress rule above; 0: threshold only
 *   block_tokens the rule (threshold and fallback) applies to every block of
 *                this many rows on its own (several blocks in one call:
 *                each commits at least one masked row); 0: the T rows are
 *                one block
 *   tokens       [T] int32          in/out: current block contents
 *   argmax       [T] int32 or NULL  receives argmax_t for every row
 *   conf         [T] fp32 or NULL   receives conf_t for every row
 *   n_committed  DEVICE int32* or NULL: number of rows committed by this call
 * Limits: T <= 2048, H multiple of 64 and <= 2048 (V unrestricted above 2).
 */
BDM_API int bdm_lm_head_unmask(const uint16_t* h, int T, int H, const uint16_t* w_head, int V,
                       int weight_layout, int32_t mask_id, float threshold, int fallback,
                       int block_tokens, int32_t* tokens, int32_t* argmax, float* conf,
                       int32_t* n_committed, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * The head in two phases, for callers that merge statistics themselves (for
 * instance over vocabulary shards held by several devices): phase 1 streams
 * one shard of the head and reduces every (token, workgroup) slice of logits
 * to an online-softmax triple; phase 2 merges any number of such triples per
 * token and applies the commit rule.  bdm_lm_head_unmask is exactly phase 1
 * over the whole vocabulary followed by phase 2.
 *
 * bdm_head_stat_parts -- number of triples per token phase 1 writes on the
 *   current device (its workgroup count).  parts: HOST pointer.
 *
 * bdm_lm_head_stats -- phase 1 over vocabulary rows [vocab_offset,
 *   vocab_offset + V) held in w_head ([V][H], weight_layout as above).  For
 *   every token t and part p < parts: stat_max[t*stat_stride + p] = the
 *   largest logit of the part's rows, stat_sum[...] = sum over those rows of
 *   exp(logit - stat_max), stat_arg[...] = the lowest vocabulary id
 *   (vocab_offset + row) holding the maximum; the row whose id equals
 *   mask_id (if it is in this shard) is left out ([files] "How it writes",
 *   step 2).  A part with no rows has max -inf, sum 0, arg INT32_MAX.
 *   stat_* are DEVICE fp32/int32 arrays of T*stat_stride elements,
 *   stat_stride >= parts; V >= 1; vocab_offset >= 0.
 *
 * bdm_unmask_from_stats -- phase 2: per token, merge stat_*[t*stat_stride +
 *   0 .. parts-1] (max of maxima; sums rescaled to the common max and added;
 *   equal maxima keep the lowest id), conf = 1/sum, argmax = that id (a row
 *   with no finite logit: -1 and conf 0, as in bdm_lm_head_unmask), then the
 *   commit rule of bdm_lm_head_unmask on tokens (same arguments, block_tokens
 *   included, and outputs).
 */
BDM_API int bdm_head_stat_parts(int* parts);

BDM_API int bdm_lm_head_stats(const uint16_t* h, int T, int H, const uint16_t* w_head, int V,
                              int vocab_offset, int weight_layout, int32_t mask_id,
                              float* stat_max, float* stat_sum, int32_t* stat_arg,
                              int stat_stride, void* stream);

BDM_API int bdm_unmask_from_stats(const float* stat_max, const float* stat_sum,
                                  const int32_t* stat_arg, int T, int parts, int stat_stride,
                                  int32_t mask_id, float threshold, int fallback,
                                  int block_tokens, int32_t* tokens, int32_t* argmax,
                                  float* conf, int32_t* n_committed, void* stream);

/*
 * bdm_lm_head_verify -- the verify epilogue of self-speculative decoding
 * ([files] "Two ways to run it"): the diffusion pass proposed T = T1 - 1
 * candidate tokens; the same model run causally over them gave T1 final
 * hidden states (row t predicts position t, row T the position after the
 * last candidate).  This call streams the head once over all T1 rows and
 * keeps the longest accepted prefix of candidates plus one new token:
 *
 *   l_t      = fp32 logits h_t . w_head^T over all V rows (never stored;
 *              no row is excluded: the causal pass has no mask token)
 *   p_t      = softmax(l_t); argmax_t = argmax_v l_t (equal: lowest id)
 *   H_t      = -sum_v p_t,v log p_t,v (nats)
 *   accept_t (t < T):
 *     rule BDM_VERIFY_EXACT:     cand[t] == argmax_t
 *     rule BDM_VERIFY_THRESHOLD: p_t(cand[t]) >= min(ratio, delta * exp(-H_t))
 *                                (the page gives ratio 0.9, delta 0.6)
 *   a row with no finite logit (or a NaN sum) has argmax -1 and accepts
 *   nothing
 *   r        = number of leading accepted candidates (0 <= r <= T)
 *   tokens_out[0..r-1] = cand[0..r-1]; tokens_out[r] = argmax_r;
 *   tokens_out[r+1..T] = -1; *n_accepted = r  (r + 1 tokens this round)
 *
 * Arguments
 *   h            [T1][H] bf16     causal-pass final hidden states
 *   w_head       [V][H] bf16      head, row-major or packed (weight_layout)
 *   cand         [T1-1] int32     DEVICE candidates (NULL allowed when T1 == 1);
 *                                 an id outside [0, V) is never accepted
 *   rule         BDM_VERIFY_EXACT or BDM_VERIFY_THRESHOLD
 *   ratio, delta finite bound parameters (used by the threshold rule)
 *   tokens_out   [T1] int32 DEVICE; n_accepted: DEVICE int32*
 *   accept       [T1-1] int32 or NULL  (1 accepted, 0 rejected, every t)
 *   argmax       [T1] int32 or NULL
 *   p_cand       [T1-1] fp32 or NULL   p_t(cand[t]) (0 for an id outside [0, V))
 *   entropy      [T1] fp32 or NULL     H_t
 * Workspace: bdm_head_verify_workspace_bytes(T1, H, V).  Limits: 1 <= T1 <=
 * 2048, H in {256, 512, 1024, 2048}, V >= 2.  All outputs are written on the
 * stream; nothing is read back to the host.
 */
#define BDM_VERIFY_EXACT      0
#define BDM_VERIFY_THRESHOLD  1
#define BDM_VERIFY_RATIO_DEFAULT 0.9f
#define BDM_VERIFY_DELTA_DEFAULT 0.6f

BDM_API int bdm_head_verify_workspace_bytes(int T1, int H, int V, size_t* bytes);

BDM_API int bdm_lm_head_verify(const uint16_t* h, int T1, int H, const uint16_t* w_head, int V,
                               int weight_layout, const int32_t* cand, int rule, float ratio,
                               float delta, int32_t* tokens_out, int32_t* n_accepted,
                               int32_t* accept, int32_t* argmax, float* p_cand, float* entropy,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * bdm_packed_weight_elems -- size of the packed copy of a [rows][cols] bf16
 * matrix: ceil(rows/16)*16*cols elements (rows padded to a multiple of 16).
 *   n: HOST pointer.  cols must be a multiple of 32.  Pure host arithmetic.
 */
BDM_API int bdm_packed_weight_elems(long rows, int cols, size_t* n);

/*
 * bdm_pack_weights -- write the BDM_LAYOUT_MFMA_TILES copy of a row-major
 * bf16 matrix src [rows][cols] into dst (bdm_packed_weight_elems elements;
 * padding rows are zero).  Tile (rg, s) of 16 rows x 32 cols is 512
 * consecutive elements: dst[((rg*(cols/32) + s)*64 + l)*8 + i] =
 * src[16*rg + l%16][32*s + 8*(l/16) + i].  A one-time preparation step for
 * the weight-streaming kernels; src and dst must not overlap.
 */
BDM_API int bdm_pack_weights(const uint16_t* src, long rows, int cols, uint16_t* dst,
                             void* stream);

/*
 * bdm_pack_gate_up -- write the gate and up matrices of a layer (both
 * row-major bf16 [rows][cols], rows = E*I or I for the shared expert, a
 * multiple of 16) into one buffer dst of 2*rows*cols elements for
 * BDM_LAYOUT_MFMA_TILES_GU: 16-row group 2g holds gate group g and group
 * 2g + 1 up group g, each in the tile order of bdm_pack_weights (a group is
 * 16*cols consecutive elements).  Pass w_gate = dst and w_up = dst +
 * 16*cols.  A one-time preparation step; gate, up and dst must not overlap.
 * Errors: BDM_ERR_INVALID_ARG for NULL pointers, rows < 16 or not a multiple
 * of 16, cols < 32 or not a multiple of 32, unaligned pointers.
 */
BDM_API int bdm_pack_gate_up(const uint16_t* gate, const uint16_t* up, long rows, int cols,
                             uint16_t* dst, void* stream);

/*
 * bdm_rmsnorm -- RMSNorm of each row, between MoE layers of a pre-norm stack.
 *   out_t = bf16( x_t / sqrt(mean(x_t^2) + eps) * gamma ), fp32 arithmetic.
 * The pages name no normalisation; this is the per-layer pre-norm of the
 * 40-layer stack workload (eps 1e-6, unit gamma).
 *   x [T][H] bf16, gamma [H] fp32 or NULL (= all ones), out [T][H] bf16
 *   (out may equal x).  H multiple of 64 and <= 2048; any T >= 1 (one
 *   workgroup per row).  Pointers 16-byte aligned.
 */
BDM_API int bdm_rmsnorm(const uint16_t* x, const float* gamma, float eps, int T, int H, uint16_t* out,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BDMOE_H */
