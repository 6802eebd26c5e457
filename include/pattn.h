/*
 * pattn.h -- C ABI of the partitioned-attention library for MI355X (gfx950).
 *
 * One operation sits at the centre: the dynamic-suffix queries of a
 * flow-matching denoising step attend over three KV regions, a pinned
 * instruction prefix, a sliding window of visual frames held in a static ring
 * buffer, and the step's own freshly computed suffix KV ("Reflex: Real-Time
 * VLA Control through Streaming Inference" paper review, §3 Architecture,
 * Eq. 1). Around it: the ring buffer itself (§3 component table; §5 Code
 * analysis), AdaRMSNorm with its conditioning MLP (§3 Eq. 2; §5 module), the
 * packed QKV projection it feeds (§2/§4: a packed-QKV kernel is one of the
 * fused operators), and the shared-KV decode readers of the OxyGen review
 * ("OxyGen: Unified KV Cache Management for Vision-Language-Action Models
 * under Multi-Task Parallelism", core method and method details).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a caller-owned DEVICE pointer, dense, in the
 *   row-major layout written next to it ([a][b][c] means c is contiguous).
 *   It must stay valid until the work queued on `stream` has finished.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call only enqueues work; nothing synchronises the device.
 * - bf16 tensors hold raw bfloat16 words; "f32" tensors IEEE binary32.
 * - No entry point allocates device memory. Scratch space is passed in as
 *   `workspace` (device, 256-byte aligned) and sized by the matching
 *   *_workspace_bytes query; its contents need no initialisation.
 * - Arguments are validated before any launch. On failure nothing is
 *   enqueued, a status other than PA_OK is returned and pa_last_error()
 *   describes it. No C++ exception ever crosses this boundary.
 * - Handles are not thread-safe: one host thread per rb_ring at a time.
 */
#ifndef PATTN_H
#define PATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_EINVAL = 1,     /* null pointer, bad enum, negative size, bad scale */
    PA_ESHAPE = 2,     /* sizes inconsistent with the ring or each other   */
    PA_ESTATE = 3,     /* call not allowed in the ring's current state     */
    PA_EDEVICE = 4,    /* a HIP runtime call failed                        */
    PA_ERANGE = 5      /* workspace too small, or a limit exceeded         */
} pa_status;
/* There is no "non-finite" status. Whether a value is NaN or Inf is only
 * known on the device after the enqueue has returned, so the calls that
 * check (the norms, the projections, the denoising step) OR bit 0 into a
 * caller-owned device word, `nonfinite`, which the caller reads when it
 * synchronises. A status describes only what the host validated. */

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Text of the last error raised on the calling thread ("" if none). */
const char* pa_last_error(void);

/* ========================================================================
 * Ring buffer (Reflex review §3 ring-buffer diagram and component table,
 * §5 ring-buffer initialisation): two zero-initialised static buffers
 *     K, V : [num_layers][P + S*F][num_kv_heads][head_dim],  S = W + spare_slots
 * Tokens [0, P) hold the pinned prefix; slot s (0 <= s < S) holds tokens
 * [P + s*F, P + (s+1)*F). Frame f is written to slot f mod S and the window
 * is the newest W frames. With S = W a push overwrites the frame pushed W
 * frames earlier: that overwrite is the eviction. The library never
 * reallocates or moves the buffers.
 *
 * A spare slot (spare_slots = 1) lets a producer fill the next frame while
 * steps on another stream still read the window (Reflex review, system
 * architecture, Figure 3: a vision thread pushes into the shared cache while
 * the policy thread denoises from it): the spare slot is never part of the
 * window, rb_stage_frame fills it, rb_commit_frame makes it the newest
 * window slot and frees the oldest, which becomes the next spare.
 * ====================================================================== */
typedef struct {
    int32_t num_layers;        /* L  > 0 */
    int32_t num_kv_heads;      /* Hkv > 0 */
    int32_t head_dim;          /* D: 32, 64, 128 or 256 (f32 rings); 64, 128 or 256 (bf16 rings) */
    int32_t pin_capacity;      /* P >= 0 */
    int32_t num_slots;         /* W > 0: frames in the sliding window */
    int32_t tokens_per_frame;  /* F > 0 */
    int32_t dtype;             /* pa_dtype of the K/V words */
    int32_t spare_slots;       /* 0, or 1 for asynchronous pushes (rb_stage_frame / rb_commit_frame) */
} rb_config;

typedef struct {
    int32_t head;              /* slot the next push writes: frames_pushed mod S */
    int32_t count;             /* frames in the window, min(frames_pushed, W) */
    int32_t pinned;            /* pinned prefix tokens (0 until rb_pin_prefix) */
    int32_t reserved;
    int64_t frames_pushed;
} rb_state;

typedef struct rb_ring rb_ring;   /* opaque; host-side metadata only */

/* Bind two caller-owned, zeroed device buffers of the layout above.
 * The handle borrows the buffers; rb_destroy frees only the handle.
 * PA_EINVAL: null argument or bad dtype; PA_ESHAPE: non-positive sizes. */
pa_status rb_create(const rb_config* cfg, void* k_buf, void* v_buf, rb_ring** out);
pa_status rb_destroy(rb_ring* ring);

/* Copy the prefix K/V, [L][n_tokens][Hkv][D], into tokens [0, n_tokens) of
 * every layer. Allowed once (PA_ESTATE on a second call); n_tokens <= P
 * (PA_ESHAPE otherwise). The prefix is computed once, at t = 0 (Eq. 1 text). */
pa_status rb_pin_prefix(rb_ring* ring, const void* k, const void* v, int32_t n_tokens, void* stream);

/* Enqueue one frame, K/V [L][F][Hkv][D]: one strided device copy into slot
 * `head` of every layer, then head = (head+1) mod S and count = min(count+1, W)
 * on the host. O(1) in the window length; no allocation. The copy is ordered
 * after earlier work on `stream` only.
 * *evicted_frame (nullable) receives the id of the frame that left the
 * window, or -1. PA_ESTATE: a staged frame is pending. */
pa_status rb_push_frame(rb_ring* ring, const void* k, const void* v, void* stream,
                        int64_t* evicted_frame);

/* Asynchronous push, step 1 (rings with a spare slot): copy the frame into
 * the spare slot on the producer's `stream`, after every step enqueued before
 * the last commit (they may still read the slot); the window is unchanged.
 * PA_ESTATE: no spare slot, or a staged frame is already pending. */
pa_status rb_stage_frame(rb_ring* ring, const void* k, const void* v, void* stream);

/* Asynchronous push, step 2: work enqueued on the consumer's `stream` after
 * this call waits for the staging copy and sees the new window (the staged
 * frame newest, the oldest frame evicted). Host metadata only besides the
 * two stream-ordered event operations. PA_ESTATE: nothing staged. */
pa_status rb_commit_frame(rb_ring* ring, void* stream, int64_t* evicted_frame);

pa_status rb_get_state(const rb_ring* ring, rb_state* out);

/* Graph capture. Attention calls plan their launches from the ring's host
 * metadata when they are enqueued, so a captured step is replayed with the
 * window as it was at capture. That stays right across later pushes when
 * the window is full (count = W) on a ring without a spare slot: the slots
 * are read in physical order whatever `head` is. On a spare-slot ring the
 * window's position moves with every commit: there the ring must keep its
 * head in a device word that the kernels read when they run.
 *   - pattn_step, pattn_step_timed, pattn_decode, pattn_fused_step and
 *     pa_denoise_step return PA_ESTATE when `stream` is capturing and the
 *     window is not full, or the ring has a spare slot and no state word.
 *   - rb_pin_prefix, rb_push_frame, rb_stage_frame, rb_commit_frame,
 *     rb_snapshot, rb_restore and rb_bind_state_word change or read host
 *     metadata at enqueue time and return PA_ESTATE under capture.
 * Replay captured steps on the stream that commits (or order them after it).
 *
 * rb_bind_state_word binds a caller-owned device buffer of four int32
 * (16-byte aligned) and writes {head, count, pinned, 0} into it on `stream`;
 * every later rb_pin_prefix, rb_push_frame, rb_commit_frame and rb_restore
 * rewrites it on its own stream, after its copies. NULL unbinds. */
pa_status rb_bind_state_word(rb_ring* ring, int32_t* state_word, void* stream);

/* ------------------------------------------------------------------------
 * Capsules (FlashRT article, PaperDaily, "FlashRT开源：27倍加速…": the
 * section on what a capsule is, and Fig. 2, the snapshot / restore / fork /
 * rollback verbs as operations on a set of static device buffers). The
 * ring's live state at a frame boundary is its valid K/V region plus the
 * metadata in rb_state. A capsule holds that region compactly: K then V,
 * each [L][pinned + count*F][Hkv][D] (per layer the pinned tokens, then the
 * first `count` slots). It may live in device memory or in host memory
 * (pinned host memory keeps the copies asynchronous).
 *   fork     = restore one capsule into several rings of the same config;
 *   rollback = restore an earlier capsule of the same ring.
 * ---------------------------------------------------------------------- */

/* Bytes of a capsule of the ring's current state (0 for a null ring). */
size_t rb_capsule_bytes(const rb_ring* ring);

/* Copy the valid region into `capsule` (stream-ordered) and return the
 * metadata in *state. PA_ERANGE: capsule_bytes < rb_capsule_bytes(). */
pa_status rb_snapshot(const rb_ring* ring, void* capsule, size_t capsule_bytes, rb_state* state,
                      void* stream);

/* Copy a capsule back into the ring's buffers (stream-ordered) and adopt
 * *state. Tokens outside the restored valid region keep whatever they held;
 * no call reads them. The ring must have the capsule's config.
 * PA_EINVAL: a state no ring of this config reaches (pinned > P, or head /
 * count not consistent with frames_pushed); PA_ERANGE: capsule too small. */
pa_status rb_restore(rb_ring* ring, const void* capsule, size_t capsule_bytes, const rb_state* state,
                     void* stream);

/* ========================================================================
 * Partitioned attention (Reflex review §3 Eq. 1; Prop. A.1):
 *     out = softmax(scale * Q [K_pin; K_slide; K_dyn]^T) [V_pin; V_slide; V_dyn]
 * for every dynamic-suffix token and query head, for layers
 * [layer_begin, layer_begin + num_layers) of the ring.
 * The cached regions are read in place: tokens [0, pinned) and the valid
 * slots [P, P + count*F) in physical slot order (softmax does not depend on
 * the order of its keys, Prop. A.1). Query head h reads KV head
 * floor(h / (n_q_heads / num_kv_heads)). The cached keys are split across
 * workgroups; each split yields a partial (max, sum, acc) that a
 * log-sum-exp combine merges in FP32. bf16 rings use bf16 MFMA with FP32
 * accumulation; f32 rings use FP32 vector arithmetic throughout.
 * ====================================================================== */
typedef struct {
    int32_t layer_begin;
    int32_t num_layers;        /* Lb >= 1 */
    int32_t n_q_heads;         /* Hq, a multiple of Hkv */
    int32_t n_dyn;             /* N >= 1 dynamic-suffix tokens */
    float   scale;             /* the 1/sqrt(d) of Eq. 1, applied once */
    int32_t out_dtype;         /* PA_F32 or PA_BF16 */
    int32_t num_splits;        /* KV splits per layer, 0..127; 0 = library's choice */
    int32_t q_layout;          /* PA_Q_TOKEN_MAJOR or PA_Q_OPERAND (bf16 rings) */
    int32_t partials_f32;      /* 0: the library's choice (bf16 partial acc on bf16 rings, FP32 on f32
                                  rings); 1: FP32 partial acc on bf16 rings too (twice the partial bytes;
                                  pattn_step / pattn_step_timed / pattn_step_noalloc only) */
} pattn_args;

/* Layouts of q for pattn_step / pattn_step_timed.
 * PA_Q_TOKEN_MAJOR: [Lb][N][Hq][D], the pages' layout.
 * PA_Q_OPERAND: the order in which the matrix-core kernel consumes Q. Query
 *   row r of KV head g is (token r / G, head g*G + r % G), G = Hq / Hkv; rows
 *   come in blocks of 32 (padded, nb = ceil(N*G / 32) blocks), and within a
 *   block the 16-dim step s holds 64 lanes x 8 dims, lane = 32 * ((d / 8) % 2)
 *   + r % 32. Element (row r, dim d) of call layer l, KV head g sits at
 *     ((((l*Hkv + g)*nb + r/32)*(D/16) + d/16)*64 + ((d/8)%2)*32 + r%32)*8 + d%8.
 *   Every wave load of Q is then 1 KB contiguous instead of 32 B from each of
 *   32 rows; a producer that writes Q (the stack's QKV projection does) can
 *   write this order at no cost. Padding rows must hold finite values (zeros
 *   from pattn_pack_q). bf16 rings only; pattn_fused_step and pattn_decode
 *   take token-major queries. */
#define PA_Q_TOKEN_MAJOR 0
#define PA_Q_OPERAND 1

/* Workspace needed by pattn_step for these arguments (0 on invalid input). */
size_t pattn_workspace_bytes(const rb_ring* ring, const pattn_args* args);

/* Bytes of q in PA_Q_OPERAND order for these arguments (0 on invalid input
 * or an f32 ring), and the conversion from token-major q (device buffers,
 * 16-byte aligned, not overlapping; asynchronous on `stream`). */
size_t pattn_operand_q_bytes(const rb_ring* ring, const pattn_args* args);
pa_status pattn_pack_q(const rb_ring* ring, const pattn_args* args, const void* q, void* q_operand,
                       void* stream);

/* q     [Lb][N][Hq][D]    ring dtype (or PA_Q_OPERAND order, args->q_layout)
 * k_dyn [Lb][N][Hkv][D]   ring dtype: K_dyn(k) of this step
 * v_dyn [Lb][N][Hkv][D]   ring dtype
 * out   [Lb][N][Hq][D]    args->out_dtype
 * PA_ESTATE: P > 0 and the prefix has not been pinned (the prefix is
 * computed once, before streaming starts). With nothing pushed yet the
 * context is [pin; suffix].
 * PA_ERANGE: ws_bytes < pattn_workspace_bytes(). */
pa_status pattn_step(const rb_ring* ring, const pattn_args* args, const void* q,
                     const void* k_dyn, const void* v_dyn, void* out,
                     void* workspace, size_t ws_bytes, void* stream);

/* pattn_step that also records ev_begin / ev_end (hipEvent_t as void*,
 * either may be NULL) on `stream` immediately before and after its split-KV
 * partial kernel, so that kernel can be timed alone while the whole step
 * runs. Same arguments, results and errors as pattn_step. */
pa_status pattn_step_timed(const rb_ring* ring, const pattn_args* args, const void* q,
                           const void* k_dyn, const void* v_dyn, void* out,
                           void* workspace, size_t ws_bytes, void* stream,
                           void* ev_begin, void* ev_end);

/* pattn_step for callers that cannot allocate device memory or pass a
 * workspace (code under graph capture that must not hold a buffer of its
 * own, tight serving loops, harnesses that forbid allocation). Same
 * arguments, results and errors as pattn_step, without the workspace: the
 * split partials go to a fixed device array of pattn_noalloc_scratch_bytes()
 * bytes (32 MiB) that the library holds on every GPU it runs on until the
 * process ends; it allocates nothing, here or later. PA_ERANGE when the call
 * needs more than that (pattn_workspace_bytes > pattn_noalloc_scratch_bytes;
 * the 18-layer long-history step with bf16 partials fits). Nothing in the
 * array needs clearing between calls: every partial a call reads it writes
 * first. All calls on one GPU share the array: calls that can overlap on one
 * GPU (different streams with no ordering between them) race on it, so
 * order them or use pattn_step. */
size_t pattn_noalloc_scratch_bytes(void);
pa_status pattn_step_noalloc(const rb_ring* ring, const pattn_args* args, const void* q,
                             const void* k_dyn, const void* v_dyn, void* out, void* stream);

/* ========================================================================
 * Shared-KV decode readers (OxyGen review, core method and method
 * details): G decode streams, one query token each, read the same cached
 * regions as the action suffix plus a private tail of their own appended
 * tokens, which no other reader sees.
 *   tail_k, tail_v : [Lb][G][tail_capacity][Hkv][D]   ring dtype
 *   tail_len       : [G] int32 (device): valid tail tokens per stream
 * ====================================================================== */
typedef struct {
    int32_t layer_begin;
    int32_t num_layers;
    int32_t n_q_heads;
    int32_t n_streams;         /* G >= 1 */
    int32_t tail_capacity;     /* >= 1 */
    float   scale;
    int32_t out_dtype;
    int32_t num_splits;        /* 0 = library's choice */
    int32_t retire_full;       /* 1: a full tail starts a new request at the next append (see below) */
} pattn_decode_args;

/* Append one token per stream, k_new/v_new [Lb][G][Hkv][D], at index
 * tail_len[g] of every layer, then tail_len[g] += 1 (on the device).
 * A request ends at a maximum length (OxyGen review, method details): with
 * args->retire_full = 1 a stream whose tail holds tail_capacity tokens has
 * finished its request, and the next request starts in its place: the new
 * token goes to index 0 and tail_len becomes 1. With retire_full = 0 a full
 * stream is left unchanged and its bit is set in *overflow_mask (device
 * uint32, nullable; bit g%32). A stream can also be retired at any time by
 * setting its tail_len to 0. tail_k, tail_v ([Lb][G][cap][Hkv][D]), k_new and
 * v_new must be 16-byte aligned (PA_EINVAL otherwise). */
pa_status pattn_append_private(const rb_ring* ring, const pattn_decode_args* args,
                               void* tail_k, void* tail_v, int32_t* tail_len,
                               const void* k_new, const void* v_new,
                               uint32_t* overflow_mask, void* stream);

size_t pattn_decode_workspace_bytes(const rb_ring* ring, const pattn_decode_args* args);

/* q [Lb][G][Hq][D]; out [Lb][G][Hq][D]. Each stream attends over
 * [pin; window; its own tail[0, tail_len[g])]. q, out, the tails and the
 * workspace must be 16-byte aligned (PA_EINVAL otherwise). */
pa_status pattn_decode(const rb_ring* ring, const pattn_decode_args* args, const void* q,
                       const void* tail_k, const void* tail_v, const int32_t* tail_len,
                       void* out, void* workspace, size_t ws_bytes, void* stream);

/* One pass for the action suffix and the decode streams together (OxyGen
 * review, core method: one shared cache read by the action expert and the
 * language expert, whose requests are batched per frame). The action rows
 * (args->n_dyn tokens x Hq heads) and the decode rows (dec->n_streams x Hq)
 * are stacked into one query matrix per layer and KV head, so the shared
 * [pin; window] keys stream once for both. Results equal pattn_step(args,
 * q, k_dyn, v_dyn, out) and pattn_decode(dec, q_dec, tails, out_dec) up to
 * rounding order: the action rows see the suffix keys and never a tail; each
 * decode row sees [pin; window; its own tail] and never the suffix. Append
 * the decode tokens first (pattn_append_private). bf16 rings only;
 * args and dec must agree on the layer range, Hq and scale (PA_EINVAL).
 * Buffers as in pattn_step and pattn_decode, all 16-byte aligned. */
size_t pattn_fused_workspace_bytes(const rb_ring* ring, const pattn_args* args,
                                   const pattn_decode_args* dec);
pa_status pattn_fused_step(const rb_ring* ring, const pattn_args* args, const void* q,
                           const void* k_dyn, const void* v_dyn, void* out,
                           const pattn_decode_args* dec, const void* q_dec, const void* tail_k,
                           const void* tail_v, const int32_t* tail_len, void* out_dec,
                           void* workspace, size_t ws_bytes, void* stream);

/* ========================================================================
 * AdaRMSNorm (Reflex review §3 Eq. 2 and component table; §5 module):
 *     y = x / sqrt(mean(x^2) + eps) * gamma,   gamma = 1 + MLP(c),
 *     c = [emb(t); state],  MLP = Linear(cond->hidden), SiLU, Linear(hidden->model)
 * emb(t) is the 128-wide sinusoid [sin(t w_i)] ++ [cos(t w_i)],
 * w_i = 10000^(-i/64). The mean of squares is taken in FP32. The MLP runs on
 * bf16 weights with c and the hidden activation rounded to bf16 and FP32
 * accumulation; gamma is kept in FP32.
 * ====================================================================== */
typedef struct {
    const void* w1;            /* bf16 [L][hidden][cond_emb + state_dim], 16-byte aligned */
    const void* b1;            /* bf16 [L][hidden] */
    const void* w2;            /* bf16 [L][model][hidden], 16-byte aligned */
    const void* b2;            /* bf16 [L][model] */
    int32_t num_layers;        /* L stacked MLPs (one per layer) */
    int32_t cond_emb;          /* 128 (any even width is accepted) */
    int32_t state_dim;         /* s, 0 <= s <= 128; cond_emb + s a multiple of 8, at most 512 */
    int32_t hidden_dim;        /* multiple of 64 in [64, 4096] */
    int32_t model_dim;         /* multiple of 64 */
} ada_mlp;

size_t ada_gamma_workspace_bytes(const ada_mlp* mlp, int32_t n_t);

/* gamma[l][i][:] = 1 + MLP_l([emb(t[i]); state]) for every layer l and
 * timestep i (a frame's ten steps in one call). t: HOST array [n_t];
 * state: device bf16 [state_dim]; gamma: device f32 [L][n_t][model_dim].
 * The state is bf16, not f32: the MLP's input c = [emb(t); state] is
 * rounded to bf16 before the first product anyway (the MLP runs in BF16),
 * so a bf16 state loses nothing and matches how a bf16 model holds it.
 * 1 <= n_t <= 16 and n_t * hidden_dim <= 32768 (a workgroup stages the n_t
 * hidden activations of its layer, 64 KB at most); other sizes, or an MLP
 * outside the limits above, return PA_ESHAPE before any launch. */
pa_status ada_gamma(const ada_mlp* mlp, const float* t, int32_t n_t, const void* state,
                    float* gamma, void* workspace, size_t ws_bytes, void* stream);

/* The whole of Eq. 2 for one layer's MLP (layer index `layer` of mlp) and one t:
 * x bf16 [rows][model_dim] -> y [rows][model_dim] in y_dtype. `workspace`
 * as sized by ada_rmsnorm_workspace_bytes. *nonfinite (device, nullable)
 * gets bit 0 set if any output is NaN or Inf. */
size_t ada_rmsnorm_workspace_bytes(const ada_mlp* mlp);
pa_status ada_rmsnorm(const void* x, int32_t rows, const ada_mlp* mlp, int32_t layer, float t,
                      const void* state, float eps, void* y, int32_t y_dtype,
                      uint32_t* nonfinite, void* workspace, size_t ws_bytes, void* stream);

/* AdaRMSNorm with a precomputed gamma (f32 [model_dim]) fused into the
 * packed QKV projection:
 *     y = bf16(x / sqrt(mean(x^2)+eps) * gamma);  [q|k|v] = y W_qkv^T
 * x bf16 [rows][model_dim]; w_qkv bf16 [(Hq + 2 Hkv) * D][model_dim]
 * (nn.Linear layout: q heads, then k heads, then v heads);
 * q bf16 [rows][Hq][D], k_dyn and v_dyn bf16 [rows][Hkv][D].
 * rows <= 64; model_dim = 128 x {2, 4, 6, 8, 12, 16}; D a multiple of 32;
 * x, gamma and w_qkv 16-byte aligned. The norm is fused into the projection
 * (every workgroup forms its A operand from x on the fly), so the workspace
 * size is 0 and `workspace` may be NULL. *nonfinite (nullable) gets bit 0 if a
 * normalised element is NaN or Inf. */
size_t ada_rmsnorm_qkv_workspace_bytes(int32_t rows, int32_t model_dim);
pa_status ada_rmsnorm_qkv(const void* x, int32_t rows, int32_t model_dim, const float* gamma,
                          float eps, const void* w_qkv, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, void* q, void* k_dyn, void* v_dyn,
                          uint32_t* nonfinite, void* workspace, size_t ws_bytes, void* stream);

/* ========================================================================
 * Layer glue of the denoising stack. The pages give none; this is a reading:
 * a residual out-projection with no bias and no FFN, the velocity taken as
 * the last layer's stream, and an Euler step of size dt:
 *     h <- bf16(h + o W_o^T)                      (residual out-projection)
 * and, when x is not NULL, the Euler update of the flow state
 *     x <- bf16(x - dt * h)                       (v = last layer's stream)
 * o bf16 [rows][in_dim]; w_o bf16 [model_dim][in_dim]; h, x bf16 [rows][model_dim].
 * rows <= 64; in_dim = 128 x {2, 4, 6, 8, 12, 16}; model_dim a multiple of 32.
 * *nonfinite (nullable) gets bit 0 if a new h or x element is NaN or Inf.
 * ====================================================================== */
pa_status oproj_residual(const void* o, const void* w_o, void* h, int32_t rows, int32_t in_dim,
                         int32_t model_dim, void* x, float dt, uint32_t* nonfinite, void* stream);

/* ========================================================================
 * FFN of the full action-expert layer. The pages name SwiGLU fusion,
 * FlashNorm and FusedAdaLN among their fused operators (Reflex review, §2
 * and the §3 system-optimisation row; Fig. 11) but do not give the layer.
 * Reading: with its own AdaRMSNorm gamma,
 *     y   = bf16(AdaRMSNorm(h, gamma))             (fused into the next GEMM)
 *     act = bf16(SiLU(y W_gate^T) * (y W_up^T))     (FP32 products, SwiGLU in the epilogue)
 *     h  <- bf16(h + act W_down^T)
 * and, when x is not NULL, the Euler update x <- bf16(x - dt * h).
 * h, x bf16 [rows][model_dim]; w_gate, w_up bf16 [ffn_dim][model_dim];
 * w_down bf16 [model_dim][ffn_dim] (nn.Linear layouts, no biases);
 * gamma f32 [model_dim]. rows <= 64; model_dim = 128 x {2, 4, 6, 8};
 * ffn_dim = 1024 x {1, 2, 3, 4, 6, 8}. The down projection is split over
 * ffn_dim: each 512-wide chunk is summed into FP32 partials, which a second
 * kernel adds in chunk order before the residual. The workspace holds act
 * and those partials (ffn_swiglu_workspace_bytes; 0 on unsupported sizes).
 * Every pointer 16-byte aligned. *nonfinite (nullable) gets bit 0 if a
 * normalised element, a new h or a new x is NaN or Inf.
 * ====================================================================== */
size_t ffn_swiglu_workspace_bytes(int32_t rows, int32_t model_dim, int32_t ffn_dim);
pa_status ffn_swiglu(void* h, int32_t rows, int32_t model_dim, int32_t ffn_dim, const float* gamma,
                     float eps, const void* w_gate, const void* w_up, const void* w_down, void* x, float dt,
                     uint32_t* nonfinite, void* workspace, size_t ws_bytes, void* stream);

/* ========================================================================
 * One denoising step of the stack, all layers (the chain the pages'
 * denoising loop runs ten times per frame; Reflex review §6 Table 7):
 *   h = x
 *   for l in layers:  [q|k|v] = ada_rmsnorm_qkv(h, gamma[l])      (Eq. 2)
 *                     o = partitioned attention, layer l           (Eq. 1)
 *                     h = bf16(h + o W_o[l]^T)
 *                     h = ffn_swiglu(h, gamma_ffn[l])             (when ffn_dim > 0)
 *   x = bf16(x - dt * h)
 * When Hq * D is a multiple of 512 the out-projection is summed like the
 * FFN's down projection (512-wide chunks of FP32 partials, added in chunk
 * order), so it can differ from oproj_residual in the last bf16 bit.
 * gamma, gamma_ffn: f32, layer l's vector at + l * gamma_layer_stride,
 * [model_dim] each (gamma_ffn may be NULL when ffn_dim = 0).
 * x: bf16 [rows][model_dim], updated in place. Layers [0, num_layers) of
 * the ring; the ring's head_dim and KV heads define D and Hkv.
 * ====================================================================== */
typedef struct {
    int32_t num_layers;
    int32_t rows;              /* N suffix tokens, <= 64 */
    int32_t model_dim;         /* 128 x {2, 4, 6, 8, 12, 16} */
    int32_t n_q_heads;
    const void* w_qkv;         /* bf16 [L][(Hq + 2 Hkv) * D][model_dim] */
    const void* w_o;           /* bf16 [L][model_dim][Hq * D] */
    float eps;
    float scale;               /* attention scale, applied once */
    float dt;                  /* Euler step */
    int32_t num_splits;        /* attention KV splits; 0 = library's choice */
    int32_t ffn_dim;           /* 0: no FFN; else 1024 x {1, 2, 3, 4, 6, 8} (model_dim <= 1024) */
    const void* w_gate;        /* bf16 [L][ffn_dim][model_dim] */
    const void* w_up;          /* bf16 [L][ffn_dim][model_dim] */
    const void* w_down;        /* bf16 [L][model_dim][ffn_dim] */
    int32_t packed;            /* 1: all five weights are fragment-packed (pa_pack_weight) */
} pa_stack;

/* Fragment-packed weights for the stack (pa_stack.packed = 1).
 * The projections of the stack have 51-64 rows and stream one weight matrix
 * each, so they are bound by how many memory requests their loads take.
 * pa_pack_weight rewrites an nn.Linear weight W bf16 [n][k] once, at setup,
 * into the order the matrix cores read it: 32-row blocks, and inside a block
 * 16-k steps of 64 lanes x 8 elements, so that every wave load is 1 KB
 * contiguous. Element (r, c) lands at
 *     (((r / 32) * (k / 16) + c / 16) * 64 + ((c / 8) % 2) * 32 + r % 32) * 8 + c % 8.
 * The packed matrix has the size of the input. Because n is a multiple of
 * 32, packing a per-layer stack [L][n][k] as one [L * n][k] matrix packs
 * each layer in place, so layer l still starts at l * n * k elements.
 * w and w_packed: device, 16-byte aligned, distinct, caller-owned; n a
 * multiple of 32, k a multiple of 16. Asynchronous on `stream`.
 * With packed = 1 the stack also needs model_dim in {512, 1024},
 * Hq * D = 1024 x {1, 2, 3, 4, 6, 8} and ffn_dim (when set) likewise; its
 * results are bit-identical to the unpacked stack's. */
pa_status pa_pack_weight(const void* w, int32_t n, int32_t k, void* w_packed, void* stream);

/* On return (in stream order) the first rows * model_dim bf16 words of the
 * workspace hold the last layer's stream h_L, the velocity of the Euler
 * step; a call with stack->num_layers = l leaves h_l there. */
size_t pa_denoise_step_workspace_bytes(const rb_ring* ring, const pa_stack* stack);
pa_status pa_denoise_step(const rb_ring* ring, const pa_stack* stack, void* x, const float* gamma,
                          const float* gamma_ffn, int64_t gamma_layer_stride, uint32_t* nonfinite,
                          void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PATTN_H */
