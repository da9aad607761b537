/*
 * w4moe -- batched-concurrent int4 (W4A16, group-wise) MoE decode step on one
 * MI355X (gfx950).  C ABI.
 *
 * The operation is one token's forward pass for B concurrent streams of a
 * packed-int4 mixture-of-experts transformer: every dense projection is applied
 * to all B rows at once, so each packed-int4 weight is read once per step; the
 * selected experts of all B streams run as one grouped operation against a
 * device-resident expert bank ("Batched-concurrent 4-bit serving on Apple
 * Silicon", section 1); attention reads a fixed KV arena through a stable
 * per-stream slot that is never wiped when the batch composition changes
 * ("Per-stream KV-slot isolation for parallel low-bit decode on Apple
 * Silicon", section 1).
 *
 * Conventions for every entry point:
 *  - Device pointers ("_dev") are caller-owned HIP device memory; the library
 *    never allocates or frees device memory.  Host pointers ("_host") are read
 *    during the call only.
 *  - fp16 data are IEEE binary16 bit patterns (uint16_t), row-major.
 *  - int4 weights arrive in the canonical layout: packed [N][K/2] bytes, byte
 *    j of a row holds element 2j in bits 0-3 and element 2j+1 in bits 4-7,
 *    each a 4-bit two's-complement code in [-8, 7]; scales [N][K/group] fp16.
 *    The dequantised weight is code * scale; y = x . W^T.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls that take a
 *    stream enqueue work on it and return; the caller synchronises.
 *  - Errors are negative status codes (W4_E_*), never traps.  Every argument
 *    is validated before anything is enqueued or any host state changes, so a
 *    failed call has no effect.  w4_last_error() gives a message.  Errors
 *    that only the device can see (a token id outside the vocabulary) are
 *    sticky: the next enqueueing call on the context, or w4_check_errors,
 *    returns them once.
 *  - One context is used by one host thread at a time; calls that enqueue on
 *    one device must not overlap in time with other calls on the same context
 *    (the batched-serving page, section 1: one submit and wait per step).
 */
#ifndef W4MOE_H
#define W4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct w4_ctx w4_ctx;

/* Model geometry.  Requirements: hidden, n_q_heads*head_dim and moe_inter are
 * multiples of 128 and at most 4096 (at most 2048 unless a multiple of 256);
 * head_dim is 64 or 128; n_q_heads is a multiple of n_kv_heads with at most
 * 16 q heads per kv head; top_k <= 16, top_k <= n_experts <= 256; group is
 * 32, 64 or 128.  The layer is the pages' MoE decoder layer: RMSNorm, fused
 * q/k/v projection, rotary, GQA attention, output projection with residual,
 * RMSNorm, top-k softmax router, SwiGLU experts, residual. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, moe_inter, vocab, group;
  float rms_eps, rope_theta;
} w4_model_desc;

enum {
  W4_OK = 0,
  W4_E_INVALID = -1,     /* bad argument or geometry, or an invalid token id seen on the device */
  W4_E_NO_SLOT = -2,     /* every slot is live */
  W4_E_CONTEXT_CAP = -3, /* prompt_len + max_new_tokens > cap, or a stream is at the cap */
  W4_E_BAD_SLOT = -4,    /* slot not live, duplicated in one call, or seeded twice */
  W4_E_NOT_READY = -5,   /* slot has a prompt that was not seeded yet */
  W4_E_HIP = -6,         /* a HIP runtime call failed (see w4_last_error) */
  W4_E_UNSUPPORTED = -7  /* device is not gfx950, or a size beyond the limits above */
};

/* Weight tensor ids for w4_bank_load. */
enum {
  W4_T_QKV = 0,      /* [(n_q + 2 n_kv) * head_dim][hidden]: q heads, then k heads, then v heads */
  W4_T_O = 1,        /* [hidden][n_q * head_dim] */
  W4_T_ROUTER = 2,   /* [n_experts][hidden] */
  W4_T_GATE = 3,     /* per expert [moe_inter][hidden] */
  W4_T_UP = 4,       /* per expert [moe_inter][hidden] */
  W4_T_DOWN = 5,     /* per expert [hidden][moe_inter] */
  W4_T_EMBED = 6,    /* [vocab][hidden] (layer ignored) */
  W4_T_LM_HEAD = 7,  /* [vocab][hidden] (layer ignored) */
  W4_T_ATTN_NORM = 8,  /* fp16 [hidden] RMSNorm gain, scales_dev unused */
  W4_T_MOE_NORM = 9,   /* fp16 [hidden] */
  W4_T_FINAL_NORM = 10 /* fp16 [hidden] (layer ignored) */
};

/* Bytes the caller must provide.  Arena: the KV store, sized by max_streams x
 * ctx_cap x geometry ("Per-stream KV-slot isolation ...", section 1: the
 * arena is keyed by the max-stream count and geometry; section 5: its
 * standing cost is reported at boot).  Bank: every weight in the library's
 * own tiled layout.  Workspace: per-step activations and scratch.  0 for a
 * geometry or size the library does not support. */
size_t w4_arena_bytes(const w4_model_desc* desc, int32_t max_streams, int32_t ctx_cap);
size_t w4_bank_bytes(const w4_model_desc* desc);
size_t w4_workspace_bytes(const w4_model_desc* desc, int32_t max_streams, int32_t ctx_cap);

/* Create a context over caller memory (sizes from the queries above; 256-byte
 * aligned).  max_streams in [1, 32]; ctx_cap a positive multiple of 64, at
 * most 16384.  W4_E_INVALID for a bad geometry or size, W4_E_UNSUPPORTED when
 * n_experts + max_streams * top_k / 16 + 1 expert work units do not fit the
 * grouped products (2 * 64 * K/256 for K = hidden and K = moe_inter).  No
 * device work is done here; *out is NULL on failure. */
int w4_create(const w4_model_desc* desc, int32_t max_streams, int32_t ctx_cap, void* arena_dev,
              void* bank_dev, void* workspace_dev, w4_ctx** out);
/* Waits for the context's enqueued work, then frees its host state. */
void w4_destroy(w4_ctx* ctx);

/* Copy one canonical tensor into the bank (repacked on the device; the
 * device-resident expert bank of the batched-serving page, section 1).
 * expert: index for W4_T_GATE/UP/DOWN, or -1 to load all experts at once from
 * [n_experts][N][K/2] / [n_experts][N][K/group]; ignored otherwise.  The
 * source buffers must stay valid until the stream reaches this work. */
int w4_bank_load(w4_ctx* ctx, int32_t layer, int32_t tensor, int32_t expert, const void* packed_dev,
                 const void* scales_dev, void* stream);

/* Slot lifecycle ("Per-stream KV-slot isolation ...", section 1: a stable
 * per-stream slot, seeded once at join, released on retire as a logical reset
 * with the buffer reused; section 5: requests over the context cap are
 * rejected at admission).
 * alloc: takes the lowest free slot; W4_E_CONTEXT_CAP when prompt_len +
 * max_new_tokens > ctx_cap, W4_E_NO_SLOT when none is free.  The slot's
 * position starts at 0.
 * seed: once per join, writes the prompt's K/V (canonical
 * [n_layers][prompt_len][n_kv][head_dim] fp16, keys already rotary-embedded)
 * into the slot and sets its position to prompt_len.  A slot allocated with
 * prompt_len > 0 cannot decode before it is seeded (W4_E_NOT_READY).
 * release: logical reset; nothing is wiped, the slot's memory is reused by the
 * next alloc.  Other slots are never touched by any of these calls. */
int w4_slot_alloc(w4_ctx* ctx, int32_t prompt_len, int32_t max_new_tokens, int32_t* slot_out);
int w4_slot_seed(w4_ctx* ctx, int32_t slot, const void* k_dev, const void* v_dev, void* stream);
int w4_slot_release(w4_ctx* ctx, int32_t slot);
/* Current position (tokens cached) of a live slot. */
int w4_slot_position(const w4_ctx* ctx, int32_t slot, int32_t* pos_out);
/* Advance the positions of n distinct live slots by one (used with the
 * per-layer entry points, which do not move positions). */
int w4_slots_advance(w4_ctx* ctx, int32_t n, const int32_t* slots_host);
/* Seed-at-join prefill ("Per-stream KV-slot isolation ...", section 1: a
 * stream's KV is seeded once, at join), through the model itself: a slot
 * allocated with prompt_len = P > 0 (and not yet seeded) gets the K/V of its
 * prompt tokens_dev int32 [P] at positions 0..P-1, computed causally layer by
 * layer over all P rows (the dense products as M = P row GEMMs, causal
 * attention over the slot, the routed experts as one grouped product per
 * layer), and its position becomes P.  Outputs: the last prompt token's fp16
 * logits [vocab] (logits_dev may be NULL), the next token id int32 [1]
 * (next_dev may be NULL; greedy, or the slot's sampling at draw counter P-1),
 * and optionally the expert ids route_ids_dev int32 [n_layers][P][top_k].
 * workspace_dev: caller-owned, 256-byte aligned, at least
 * w4_prefill_workspace_bytes(desc, P, ctx_cap) bytes (ws_bytes gives its
 * size).  Limits: P * top_k <= 16384 and n_experts * ceil(P / 32) * 6 <=
 * 61440 (W4_E_UNSUPPORTED beyond).  An out-of-range token id is
 * reported like the decode step's (sticky W4_E_INVALID).  The call replaces
 * w4_slot_seed for that slot. */
size_t w4_prefill_workspace_bytes(const w4_model_desc* desc, int32_t max_prompt, int32_t ctx_cap);
int w4_slot_prefill(w4_ctx* ctx, int32_t slot, const int32_t* tokens_dev, void* workspace_dev, size_t ws_bytes,
                    void* logits_dev, int32_t* next_dev, int32_t* route_ids_dev, void* stream);

/* Sampling of a live slot's next tokens (beyond the pages' greedy decoding;
 * the batched-serving page, section 5, names non-greedy sampling as not
 * validated there).  temperature 0 (the default after w4_slot_alloc) is
 * greedy; otherwise: rank ids by (logit descending, id ascending), keep the
 * first top_k (1..64), weight rank r by exp((l_r - l_0) / temperature), keep
 * the shortest prefix whose running sum reaches top_p (0 < top_p <= 1) of the
 * total, and invert that prefix's running sums at a draw u in [0, 1): u is
 * the top 24 bits of output number p of the SplitMix64 generator started at
 * seed, p the slot's position when the token is decoded.  So a stream's
 * tokens depend on its own seed and positions only, never on the batch.
 * W4_E_BAD_SLOT / W4_E_INVALID on a bad slot or parameter. */
int w4_slot_set_sampling(w4_ctx* ctx, int32_t slot, uint64_t seed, float temperature, int32_t top_k,
                         float top_p);
/* Diagnostic, the inverse of w4_slot_seed: the K/V a live, seeded slot holds
 * at positions 0 .. p-1 (p = its current position) -> k_dev, v_dev, each
 * canonical [n_layers][p][n_kv][head_dim] fp16 (post-rotary keys), caller-
 * owned with room for that many elements.  Nothing is written when p = 0. */
int w4_slot_read_kv(w4_ctx* ctx, int32_t slot, void* k_dev, void* v_dev, void* stream);

/* One decode step for B streams ("Batched-concurrent 4-bit serving ...",
 * section 1: all layers and the output projection of the B streams in one
 * submission; section 3: greedy decoding, or each slot's sampling as set by
 * w4_slot_set_sampling).  Row b is the stream in
 * slots_host[b] at its current position p_b.  tokens_dev int32 [B] input ids
 * (an id outside [0, vocab) gives a zero embedding row and a sticky
 * W4_E_INVALID from the next enqueueing call or w4_check_errors).  Writes the
 * new K/V at p_b of each slot, returns fp16 logits [B][vocab] (logits_dev may
 * be NULL) and the next ids int32 [B] (greedy: ties to the lower id).
 * route_ids_dev: optional int32 [n_layers][B][top_k] expert ids per rank.
 * On success every listed slot's position advances by one.  A row's result
 * is bit-identical whatever the other rows, their order and the slot ids
 * (same page, section 3: a stream's output is the same alone or batched). */
int w4_decode_step(w4_ctx* ctx, int32_t B, const int32_t* slots_host, const int32_t* tokens_dev,
                   void* logits_dev, int32_t* next_dev, int32_t* route_ids_dev, void* stream);

/* Wait for every step enqueued on the context, then return W4_E_INVALID once
 * if one of them was given a token id outside [0, vocab) since the last
 * report (W4_OK otherwise). */
int w4_check_errors(w4_ctx* ctx);

/* ---- per-stage entry points (same kernels as w4_decode_step) ---- */

/* Dense W4A16 product with a bank tensor ("Batched-concurrent ...", section
 * 1: one batched 4-bit GEMM reads each packed-int4 weight once across the B
 * rows): y = x . dequant(W)^T, fp32 accumulation.  x fp16 [B][K]; y fp16
 * [B][N], except W4_T_ROUTER which writes fp32 [B][n_experts].  expert
 * selects one expert of GATE/UP/DOWN.  B in [1, max_streams]. */
int w4_gemm(w4_ctx* ctx, int32_t layer, int32_t tensor, int32_t expert, int32_t B, const void* x_dev,
            void* y_dev, void* stream);

/* Top-k softmax routing and (stream, expert) bucketing for B streams (the
 * grouped expert dispatch of the batched-serving page, sections 1 and 3).
 * logits fp32 [B][n_experts] -> ids int32 [B][top_k] (ranked by logit,
 * ties to the lower id), w fp32 [B][top_k] (softmax over the selected),
 * counts int32 [n_experts], offsets int32 [n_experts + 1], and the pairs
 * ordered by (expert, stream): pair_stream, pair_rank int32 [B * top_k].
 * Any output pointer except ids and w may be NULL. */
int w4_route(w4_ctx* ctx, int32_t B, const float* logits_dev, int32_t* ids_dev, float* w_dev,
             int32_t* counts_dev, int32_t* offsets_dev, int32_t* pair_stream_dev,
             int32_t* pair_rank_dev, void* stream);

/* MoE block of one layer for B rows, no residual (the selected experts of all
 * streams as one grouped operation against the expert bank, batched-serving
 * page, section 1): y = sum_r w_r * expert_r(x) with SwiGLU experts.  x fp16
 * [B][hidden] is the block's (normalised) input.  router_logits_dev fp32
 * [B][n_experts], or NULL to compute them from x with the layer's router.
 * route_ids_dev optional int32 [B][top_k]. */
int w4_moe(w4_ctx* ctx, int32_t layer, int32_t B, const void* x_dev, const float* router_logits_dev,
           void* y_dev, int32_t* route_ids_dev, void* stream);

/* Slot-indexed GQA decode attention of one layer ("Per-stream KV-slot
 * isolation ...", section 1: each stream reads and appends its own slot):
 * q fp16 [B][n_q][head_dim] (already rotary-embedded), k_new / v_new fp16
 * [B][n_kv][head_dim] are written at each slot's current position p_b, then
 * attention over 0..p_b -> o fp16 [B][n_q][head_dim].  Positions do not move. */
int w4_attn_decode(w4_ctx* ctx, int32_t layer, int32_t B, const int32_t* slots_host, const void* q_dev,
                   const void* k_new_dev, const void* v_new_dev, void* o_dev, void* stream);

/* One decoder layer for B streams at their current positions (the
 * batched-serving page, section 1): h fp16 [B][hidden] residual stream,
 * updated in place.  Positions do not move.  route_ids_dev optional int32
 * [B][top_k]. */
int w4_layer_step(w4_ctx* ctx, int32_t layer, int32_t B, const int32_t* slots_host, void* h_dev,
                  int32_t* route_ids_dev, void* stream);

/* ---- allocation-free routing (no context) ----
 * For callers that cannot allocate device memory or hold a context (code
 * under HIP graph capture, tight serving loops): the routing and bucketing of
 * w4_route, with the same arguments and results, for B <= 32 rows of
 * n_experts <= 256 logits and top_k <= 16.  Its scratch is a 32 KiB
 * file-scope device array (one per GPU, held until the process ends), so it
 * allocates nothing; calls that overlap on one GPU share that array and race,
 * so serialise them (one stream, or events).  W4_E_UNSUPPORTED beyond those
 * sizes, W4_E_INVALID for null logits, ids or w; the message is
 * w4_last_error(NULL). */
int w4_route_noalloc(int32_t B, int32_t n_experts, int32_t top_k, const float* logits_dev, int32_t* ids_dev,
                     float* w_dev, int32_t* counts_dev, int32_t* offsets_dev, int32_t* pair_stream_dev,
                     int32_t* pair_rank_dev, void* stream);

/* ---- diagnostics ---- */
const char* w4_status_string(int32_t status);
/* Message of the context's last failure; with NULL, that of the last failed
 * context-free call on this thread. */
const char* w4_last_error(const w4_ctx* ctx);
/* Kernel launches and host-device synchronisations issued by the last
 * w4_decode_step (the batched-serving page, sections 3 and 4, counts GPU
 * submissions per token; the library itself never synchronises inside a step
 * while fewer than eight steps are in flight). */
int w4_last_step_counts(const w4_ctx* ctx, int32_t* launches, int32_t* syncs);

/* Streaming-read ceiling probe (a measurement aid, not part of the step):
 * reads src_dev[0 .. bytes) once with the 16-byte loads the weight kernels
 * use, plain (nontemporal 0) or non-temporal (1), from `grid` 256-thread
 * work-groups; sink_dev: caller-owned int32 [grid], almost never written.
 * bytes a positive multiple of 16, src_dev 16-byte aligned; W4_E_INVALID
 * otherwise.  Time it with events on `stream`. */
int w4_read_probe(const void* src_dev, size_t bytes, void* sink_dev, int32_t grid, int32_t nontemporal,
                  void* stream);

/* Context options (a verification and measurement aid; the defaults are the
 * fast path).  W4_OPT_FUSED_MOE, default 0: the grouped expert products of a
 * layer as two launches.  1: as one launch, the down product's tiles starting
 * on compute units whose gate/up share is done (per-unit completion counters
 * with bounded device-side waits; a wait that runs out is reported as
 * W4_E_HIP by the next enqueueing call or w4_check_errors); measured slower
 * than two launches at B >= 4 and equal at B = 1 on MI355X.  The results are
 * the same bit for bit.  The fused form applies where the gate/up reduction
 * length is at most 2048 and the down product's is at most the gate/up's.
 * W4_E_INVALID for an unknown option or value. */
enum { W4_OPT_FUSED_MOE = 1 };
int w4_set_option(w4_ctx* ctx, int32_t option, int32_t value);

/* Device-wide barrier probe (a measurement aid, not part of the step): the
 * cost of a phase boundary inside one persistent launch against that of a
 * launch boundary.  mode 0: n barriers among `grid` co-resident 512-thread
 * work-groups in one launch (two-level device-scope counters, bounded waits;
 * a wait that runs out sets word 1 of scratch); grid must not exceed the
 * work-groups the device keeps resident.  mode 1: n back-to-back launches of
 * an empty kernel of the same shape.  scratch_dev: caller-owned, at least
 * 2304 bytes.  W4_E_INVALID for bad arguments.  Time it with events on `stream`. */
int w4_sync_probe(int32_t mode, int32_t grid, int32_t n, void* scratch_dev, size_t bytes, void* stream);

/* Kernel families that w4_profile_begin can time. */
enum {
  W4_K_DENSE = 1,      /* dense W4A16 products: q/k/v, o, output projection */
  W4_K_MOE_GATEUP = 2, /* grouped expert gate/up + SwiGLU */
  W4_K_MOE_DOWN = 3,   /* grouped expert down */
  W4_K_ATTENTION = 4,  /* split-KV decode attention (one launch, split combine included) */
  W4_K_ROUTER = 5,     /* MoE front end: norm, router product, top-k, bucketing (one launch) */
  W4_K_MOE = 6         /* grouped expert products in one launch (gate/up + SwiGLU, then down) */
};
/* Record a HIP event pair around every launch of one kernel family in the
 * calls that follow (on the stream each call is given), until
 * w4_profile_end, which waits for the last event and returns the summed
 * kernel time in milliseconds and the number of launches timed. */
int w4_profile_begin(w4_ctx* ctx, int32_t kernel);
int w4_profile_end(w4_ctx* ctx, double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* W4MOE_H */
