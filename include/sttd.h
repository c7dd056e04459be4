/*
 * sttd.h - C ABI of the MI355X (gfx950) Qwen3-style decoder-block library.
 *
 * The operation is the shared causal-LM block that transcribe.cpp's
 * Qwen3-ASR and Canary-Qwen handlers drive in a prefill and a per-token
 * step loop (Qwen3-ASR decoder page, transcribe-cpp-sys 0.2.0,
 * src/arch/qwen3_asr/decoder.cpp: file header, build_prefill_graph,
 * build_step_graph). One block is pre-LN RMSNorm, grouped-query attention
 * with per-head Q/K RMSNorm, NeoX RoPE, a KV-cache write then read, the
 * output projection with a residual add, and SwiGLU on one packed gate_up
 * projection followed by the down projection with a residual add. After
 * the stack: a final RMSNorm, the tied lm_head and a greedy argmax.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host). Structs passed by
 *    pointer are host structs; sttd_block_weights holds device pointers.
 *  - The caller owns weights, activations, positions, ids and logits.
 *    The library owns what sttd_kv_cache_alloc / sttd_workspace_alloc
 *    allocate until the matching free.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return without synchronising. They make no host read of
 *    device data, so the block, step and head calls can be captured in a
 *    HIP graph.
 *  - Host-visible arguments are validated before anything is enqueued.
 *    Invalid arguments return an error and enqueue nothing. Device-resident
 *    values (positions, slab ids, token ids) cannot be checked on the host:
 *    kernels check them, skip the out-of-range row, and record an error
 *    code in the workspace (sttd_workspace_error reads it).
 *  - A launch failure returns STTD_ERR_BACKEND. No C++ exception crosses
 *    the ABI. Two calls that touch one KV cache or one workspace must be
 *    ordered (same stream); distinct handles are independent.
 *
 * Weight layout (row-major, [out, in]; no biases - the block's ten weight
 * slots, to_block_view on the decoder page):
 *   attn_norm[H]  wq[nq*d, H]  wk[nkv*d, H]  wv[nkv*d, H]
 *   q_norm[d]  k_norm[d]  (one gain vector shared by all heads)
 *   wo[H, nq*d]  ffn_norm[H]
 *   w_gate_up[2*I, H]: rows 0..I-1 are the gate, rows I..2I-1 the up
 *     projection (the packed tensor of pack_gate_up, Qwen3-ASR model page,
 *     load(); the row order is this ABI's contract)
 *   w_down[H, I]
 * Every matrix and gain has the storage type `wtype` (STTD_BF16 or STTD_F32).
 * Hidden states x are fp32 [rows, H], row-major.
 */
#ifndef STTD_H
#define STTD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STTD_OK = 0,
    STTD_ERR_INVALID_ARG = 1,  /* null pointer, bad size, layer/slab out of range */
    STTD_ERR_OOM = 2,          /* device allocation failed */
    STTD_ERR_BACKEND = 3,      /* a HIP call or kernel launch failed */
    STTD_ERR_CONTEXT_FULL = 4, /* positions would pass the cache's n_ctx */
    STTD_ERR_UNSUPPORTED = 5   /* shape or dtype combination not built */
} sttd_status;

typedef enum { STTD_F32 = 0, STTD_BF16 = 1, STTD_F16 = 2 } sttd_dtype;

/* Block shape (to_block_params on the decoder page). head_dim must be 64 or
 * 128; n_heads / n_kv_heads one of 1, 2, 4, 8; hidden and ffn multiples of
 * 64; hidden, ffn and n_heads * head_dim at most 8192 (else
 * STTD_ERR_UNSUPPORTED). */
typedef struct {
    int32_t hidden, n_heads, n_kv_heads, head_dim, ffn;
    float rms_eps;    /* RMSNorm epsilon, inside the square root */
    float rope_theta; /* NeoX RoPE base: pair i turns by pos * theta^(-2i/d) */
    sttd_dtype wtype; /* STTD_BF16 or STTD_F32 */
} sttd_block_params;

/* Host struct of device pointers to one block's ten weight tensors. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *ffn_norm, *w_gate_up, *w_down;
} sttd_block_weights;

typedef struct sttd_kv_cache sttd_kv_cache;   /* opaque */
typedef struct sttd_workspace sttd_workspace; /* opaque */

/* Device-side error codes recorded in a workspace (sttd_workspace_error). */
#define STTD_DEVERR_POSITION 1u /* a position was < 0 or >= the cache's n_ctx */
#define STTD_DEVERR_SLAB 2u     /* a slab id was < 0 or >= the cache's n_seq */
#define STTD_DEVERR_TOKEN 4u    /* a token id was < 0 or >= vocab */
#define STTD_DEVERR_SYNC 8u     /* a single-row projection + attention hand-off timed out (200 ms); its outputs are invalid */
#define STTD_DEVERR_ROW 16u     /* a head row index was < 0 or >= n_x_rows */

/* block_prefill flag: the FFN (and so the block output) is computed for the
 * last row only; rows 0..T-2 of x are left holding the attention residual
 * h = x + o * Wo^T. The slice_last_before_ffn option of the decoder page's
 * build_prefill_graph, for the stack's last block. */
#define STTD_LAST_ROW_FFN_ONLY 1u

const char *sttd_status_string(sttd_status s);

/* ---------------------------------------------------------------- KV cache
 * One K and one V slab per (layer, sequence): kv_init / kv_init_batched on
 * the Qwen3-ASR model page (run(), run_batch()) size it as n_ctx rows of
 * n_kv_heads * head_dim per layer; one token holds
 * n_kv_heads * head_dim * n_layers * 2 elements (load(), session limits).
 * Layout: [layer][seq][kv_head][n_ctx][head_dim], K and V in two buffers.
 * The row index of a token is its position. kv_type: STTD_F16 or STTD_F32.
 * The memory is zeroed at allocation. */
sttd_status sttd_kv_cache_alloc(int n_layers, int n_seq, int n_ctx, int n_kv_heads, int head_dim,
                                sttd_dtype kv_type, sttd_kv_cache **out /* host */);
sttd_status sttd_kv_cache_free(sttd_kv_cache *kv);
/* Cache context for a session that needs `needed` positions (prompt plus
 * generation budget), the sizing rule described in run() on the MOSS page:
 * short inputs keep the 1024 / 2048 / 4096 buckets, longer ones grow in steps
 * of 4096 (so crossing 32K does not jump to the full 131072-token worst case),
 * and the result is clamped to `ceiling`. Host function, no device work.
 * Returns 0 when needed < 1 or ceiling < 1. */
int sttd_kv_context_for(int needed, int ceiling);
/* Zero every slab (the buffer clear before a fresh prefill, run() on the
 * Qwen3-ASR model page). Enqueued as a fill kernel on `stream`. */
sttd_status sttd_kv_cache_clear(sttd_kv_cache *kv, void *stream);
/* Device pointers to the K and V slab of (layer, seq) and its element strides
 * between kv heads and between positions. For tests and fills. */
sttd_status sttd_kv_cache_view(const sttd_kv_cache *kv, int layer, int seq, void **k /* host */,
                               void **v /* host */, int64_t *head_stride /* host */,
                               int64_t *pos_stride /* host */);

/* ---------------------------------------------------------------- workspace
 * Scratch for the block and head calls (projections, attention partials,
 * argmax slots, the RoPE table), sized for up to max_rows rows per call,
 * positions < max_pos and a vocabulary of up to `vocab` rows (0: no head).
 * The RoPE table is computed on the host in fp64 and stored in fp32:
 * cos and sin of pos * theta^(-2i/d) for i < d/2. Allocating it is a
 * synchronous call. */
sttd_status sttd_workspace_alloc(const sttd_block_params *p /* host */, int max_rows, int max_pos, int vocab,
                                 sttd_workspace **out /* host */);
sttd_status sttd_workspace_free(sttd_workspace *ws);
/* Workspace options (sttd_workspace_set_option). */
/* STTD_OPT_ACT_SPLIT, default 15: precision of the activations that feed the
 * bf16-weight MFMA projections. A split activation is carried as two bf16
 * parts, hi = bf16(v) and lo = bf16(v - hi), so the product sees about 16
 * significant bits of it at twice the MFMA work. Up to 512 rows per call all
 * four are split whatever the value (those GEMMs are bound by weight bytes
 * there, so the second MFMA pass is free). Above 512 rows an activation is
 * split when its bit is set in `value` and rounded to plain bf16 otherwise:
 * STTD_SPLIT_QKV (the attention RMSNorm output), STTD_SPLIT_O (the attention
 * output), STTD_SPLIT_GATE_UP (the FFN RMSNorm output), STTD_SPLIT_DOWN (the
 * SwiGLU output). Measured on the 28-block 1.7B-shaped stack (8 packed
 * prompts of 153 rows, 1224 rows per call) against the fp64 oracle: with all
 * four plain the final logits move by 11% of their RMS, beyond the 3e-2
 * bound on hidden states; all four split, 1.2%; only the attention output or
 * only the Q|K|V input plain, 4.2% and 7.1%.
 * One block stays within the bound with all four plain (its 4096-row parity
 * test), so a caller running a single block or a shallow stack may set 0 to
 * halve the MFMA work of long prefills. */
#define STTD_OPT_ACT_SPLIT 2
#define STTD_SPLIT_QKV 1
#define STTD_SPLIT_O 2
#define STTD_SPLIT_GATE_UP 4
#define STTD_SPLIT_DOWN 8
/* STTD_OPT_QKV_ATTN, default 1: a single-row block_step with bf16 weights, an
 * f16 cache, head_dim 128, groups of 1 or 2 query heads per KV head, hidden up
 * to 4096 and attention splits of at most 128 cache rows runs its Q|K|V
 * projection and its attention as one launch: the projection's workgroups
 * publish each column as a 64-bit word tagged with a per-launch number, and
 * the attention workgroups, which start with them, fetch their cache rows and
 * then poll their head's words (a poll gives up after 200 ms and records
 * STTD_DEVERR_SYNC). The arithmetic is that of the two-launch form (value
 * 0): from the same cache state the results are bit-identical. Measured on
 * the 28-block 1.7B-shaped greedy job: 1.077 -> 1.066 ms per token. Calls
 * that share a workspace must not run concurrently. */
#define STTD_OPT_QKV_ATTN 3
/* Sets `option` to `value`. Unknown option or value: STTD_ERR_INVALID_ARG. */
sttd_status sttd_workspace_set_option(sttd_workspace *ws, int option, int value);

/* Synchronising read of the device error bits (STTD_DEVERR_*) recorded since
 * the last call, which also clears them. Not for use under graph capture. */
sttd_status sttd_workspace_error(sttd_workspace *ws, uint32_t *bits /* host */);

/* ---------------------------------------------------------------- calls */

/* Token-embedding gather (ggml_get_rows on the tied table in the decoder
 * page's build_step_graph): x[b, :] = fp32(embed[ids[b], :]) for b < B.
 * embed [vocab, hidden] of storage type wtype; ids [B] int32; x [B, hidden].
 * A device id outside [0, vocab) writes a zero row and records
 * STTD_DEVERR_TOKEN when ws is non-NULL. */
sttd_status sttd_embed_gather(const void *embed, sttd_dtype wtype, int vocab, int hidden, int B,
                              const int32_t *ids, float *x, sttd_workspace *ws, void *stream);

/* Prompt/audio injection before the first block: the elementwise blend of the
 * batched prefill graphs on the Qwen3-ASR model page (build_prefill_graph_batched:
 * x = x * keep_mask + audio_dense) and of the MOSS page (build_injection and
 * its chunked prefill): x[t, :] = embed[ids[t], :] * keep[t] + audio_dense[t, :]
 * for t < T. ids [T] int32; keep [T] fp32 (the pages put 0 at the audio
 * positions and 1 elsewhere); audio_dense [T, hidden] fp32 (the encoder's rows
 * scattered to the audio positions, zero elsewhere); x [T, hidden] fp32 out.
 * With one contiguous audio block this equals the 3-way concat of prefix
 * embeddings, audio rows and suffix embeddings in the single-sequence
 * build_prefill_graph. A device id outside [0, vocab) contributes a zero row
 * and records STTD_DEVERR_TOKEN when ws is non-NULL. */
sttd_status sttd_embed_inject(const void *embed, sttd_dtype wtype, int vocab, int hidden, int T,
                              const int32_t *ids, const float *keep, const float *audio_dense, float *x,
                              sttd_workspace *ws, void *stream);

/* Causal prefill of T rows of one sequence through one block
 * (causal_lm::block_prefill as called by build_prefill_graph).
 * Row t sits at position pos0 + t; its K and V are written at cache row
 * pos0 + t of slab `seq` in layer `layer`; it attends cache rows
 * [0, pos0 + t] (rows below pos0 must hold earlier positions, e.g. an
 * earlier chunk). x [T, hidden] fp32 is read and overwritten with the
 * block output (see STTD_LAST_ROW_FFN_ONLY). Requires 1 <= T <= the
 * workspace's max_rows; pos0 + T > n_ctx returns STTD_ERR_CONTEXT_FULL. */
sttd_status sttd_block_prefill(const sttd_block_params *p, const sttd_block_weights *w, sttd_workspace *ws,
                               sttd_kv_cache *kv, int layer, int seq, int pos0, int T, float *x, uint32_t flags,
                               void *stream);

/* Causal prefill of n sequences through one block in one call: the batched
 * prefill of the Qwen3-ASR model page (run_batch: build_prefill_graph_batched
 * over block_prefill_batched), with the prompts packed back to back instead of
 * padded to the longest. Sequence i (host arrays, i < n <= 64) has T[i] >= 1
 * rows at positions pos0[i] .. pos0[i] + T[i] - 1 in slab seq[i] (distinct);
 * its rows attend only cache rows [0, position] of its own slab (rows below
 * pos0[i] must hold earlier positions). x [sum T[i], hidden] fp32 holds the
 * sequences' rows in order and is overwritten with the block outputs. The
 * projections run once over all rows, so the weights are read once for the
 * batch. sum T[i] <= the workspace's max_rows; pos0[i] + T[i] > n_ctx:
 * STTD_ERR_CONTEXT_FULL; n outside [1, 64], a bad or repeated slab, T[i] < 1
 * or pos0[i] < 0: STTD_ERR_INVALID_ARG. */
sttd_status sttd_block_prefill_batched(const sttd_block_params *p, const sttd_block_weights *w, sttd_workspace *ws,
                                       sttd_kv_cache *kv, int layer, int n, const int32_t *seq /* host */,
                                       const int32_t *pos0 /* host */, const int32_t *T /* host */, float *x,
                                       void *stream);

/* One decode step of B rows through one block (causal_lm::block_step and
 * block_step_batched in build_step_graph / build_step_graph_batched).
 * Row b is at position pos[b] (device int32 [B]) of slab seq[b] (device
 * int32 [B], or NULL for slab b); rows must name distinct slabs. Its K, V
 * go to cache row pos[b]; it attends rows [0, pos[b]]. pos_bound (host) is
 * an upper bound on every pos[b] + 1 (<= n_ctx) used to size the launch;
 * the work done follows the actual pos[b]. x [B, hidden] fp32 in/out.
 * 1 <= B <= max_rows. pos[b] = -1 marks a row whose greedy loop has stopped
 * (sttd_greedy_stop): its attention and cache write are skipped and its
 * output row is undefined. */
sttd_status sttd_block_step(const sttd_block_params *p, const sttd_block_weights *w, sttd_workspace *ws,
                            sttd_kv_cache *kv, int layer, int B, const int32_t *seq, const int32_t *pos,
                            int pos_bound, float *x, void *stream);

/* Final RMSNorm, tied lm_head and greedy argmax over B rows (the tail of
 * build_step_graph; the host argmax in run() on the Qwen3-ASR model page
 * keeps the lowest index on ties, and so does this call; a NaN logit never
 * wins: it ranks below every number, -inf included, so a row of NaN logits
 * gives id 0). final_norm [hidden], embed [vocab, hidden] (storage wtype).
 * Input rows: with x_rows NULL, row b is read at x + b * x_row_stride
 * (floats), so the last prefill row can be passed directly. With x_rows
 * (device int32 [B]), row b is read at x + x_rows[b] * x_row_stride: the
 * per-sequence last-row gather of the batched prefill graph
 * (build_prefill_graph_batched on the Qwen3-ASR decoder page gathers each
 * utterance's last position before the final norm and head; run_batch on the
 * model page fills those positions), so ragged packed prompts take one head
 * call. n_x_rows (host) is the number of rows x holds and must be >= 1 then;
 * an index outside [0, n_x_rows) reads row 0 and records STTD_DEVERR_ROW (that
 * row's outputs are then meaningless). Outputs: ids [B] int32; optional logits
 * [B, vocab] fp32 (NULL: not written); optional next_x [B, hidden] fp32 =
 * embed[ids[b]] (the next step's input rows); optional pos [B] int32
 * incremented by one after the step (device-resident step counter). */
sttd_status sttd_lm_head_argmax(const void *final_norm, const void *embed, sttd_dtype wtype, int vocab, int hidden,
                                float rms_eps, sttd_workspace *ws, int B, const float *x, int64_t x_row_stride,
                                const int32_t *x_rows, int n_x_rows, int32_t *ids, float *logits, float *next_x,
                                int32_t *pos, void *stream);

/* The same head for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the call allocates nothing and calls no allocating
 * routine. Its scratch (the argmax keys of at most
 * STTD_STATIC_HEAD_MAX_ROWS rows and their normed bf16 planes, 256 KiB) is
 * a static device array the library holds on each GPU it runs on until the
 * process ends; its address is looked up once per device on the first call.
 * Arguments and results are those of sttd_lm_head_argmax, with the same
 * kernels, except: B > STTD_STATIC_HEAD_MAX_ROWS returns
 * STTD_ERR_INVALID_ARG; device-side error bits (STTD_DEVERR_ROW,
 * STTD_DEVERR_TOKEN) are OR'd into the optional device word `err` (NULL: not
 * recorded). Nothing in the scratch needs to start at zero. Every call on one
 * GPU shares that GPU's scratch: two calls that overlap in time on one GPU
 * (different streams, or different host threads without ordering) race and
 * give undefined results. */
#define STTD_STATIC_HEAD_MAX_ROWS 16
sttd_status sttd_lm_head_argmax_static(const void *final_norm, const void *embed, sttd_dtype wtype, int vocab,
                                       int hidden, float rms_eps, int B, const float *x, int64_t x_row_stride,
                                       const int32_t *x_rows, int n_x_rows, int32_t *ids, float *logits,
                                       float *next_x, int32_t *pos, uint32_t *err, void *stream);

/* Greedy stopping rules on the device, per row (the step loop of run() on
 * the Qwen3-ASR model page, and per row in its batched step loop): a row goes
 * on while its newest token is not eos_id, it has fewer than max_new tokens
 * and its next input position is inside the context (position + 1 <= n_ctx);
 * a row that stops for another reason than EOS is truncated. The repetition
 * guard of the MOSS page is not defined on the pages and is not applied.
 * Call it after each sttd_lm_head_argmax, whose pos argument must then be
 * NULL: this call owns the positions. State (device int32 [B], set by the
 * caller before the first call): active = 1, n_gen = 0, truncated = 0,
 * pos = the prompt length (the first step's input position). For each active
 * row b the chosen ids[b] is stored at tokens[b * max_new + n_gen[b]] and
 * n_gen[b] is incremented; with advance = 1 (every call after a decode step;
 * 0 for the call after the prefill) pos[b] moves on by one. A row that stops
 * gets active 0, truncated = (ids[b] != eos_id) and pos = -1, which marks it
 * for sttd_block_step to skip (no cache write, no error; its outputs are
 * undefined). Inactive rows are left unchanged. n_active (device int32 [1],
 * may be NULL) receives the number of rows still active. The call is
 * graph-capturable, so the whole loop can be replayed and the host reads
 * n_active between replays. */
typedef struct {
    int32_t eos_id, max_new, n_ctx;
} sttd_stop_rules;
sttd_status sttd_greedy_stop(const sttd_stop_rules *r /* host */, int B, const int32_t *ids, int advance,
                             int32_t *pos, int32_t *active, int32_t *n_gen, int32_t *tokens, int32_t *truncated,
                             int32_t *n_active, void *stream);

/* ---------------------------------------------------------------- per-kernel timing
 * The per-op profiler of the MOSS-Transcribe-Diarize page (src/arch/moss/
 * model.cpp, run() and its OpProf table: wall time per graph node), as HIP
 * events: while a kernel family's bit (1 << kind) is set in the mask, every
 * kernel an eager call of that family launches carries a start/stop event pair
 * bound to its dispatch (hipExtLaunchKernel), so each pair times one kernel
 * from dispatch to completion, as rocprofv3's kernel trace does, without the
 * gaps between kernels. Launches on a capturing stream are not timed.
 * sttd_profile_read synchronises on the recorded events and returns the number
 * of timed calls of the family and the summed milliseconds of their kernels,
 * then clears that family. A call may launch several kernels: the attention-
 * rows family spans the split kernel and its combine, the head its finalize
 * pass. */
typedef enum {
    STTD_KERN_RMSNORM = 0,      /* RMSNorm rows to bf16 (prefill) */
    STTD_KERN_QKV_GEMV = 1,     /* fused RMSNorm + Q|K|V projection, decode rows */
    STTD_KERN_QKV_GEMM = 2,     /* Q|K|V projection, MFMA */
    STTD_KERN_QK_ROPE_KV = 3,   /* per-head Q/K RMSNorm + RoPE + KV write */
    STTD_KERN_ATTN_ROWS = 4,    /* split-K attention of independent rows + combine */
    STTD_KERN_ATTN_PREFILL = 5, /* causal flash prefill attention, MFMA */
    STTD_KERN_O_GEMV = 6,       /* O projection + residual, decode rows */
    STTD_KERN_O_GEMM = 7,
    STTD_KERN_GATEUP_GEMV = 8,  /* fused RMSNorm + gate_up + SwiGLU, decode rows */
    STTD_KERN_GATEUP_GEMM = 9,
    STTD_KERN_DOWN_GEMV = 10,   /* down projection + residual, decode rows */
    STTD_KERN_DOWN_GEMM = 11,
    STTD_KERN_LM_HEAD = 12,     /* final RMSNorm + tied head + argmax */
    STTD_KERN_QKV_ATTN = 13,    /* single decode row: Q|K|V projection + attention in one launch (STTD_OPT_QKV_ATTN) */
    STTD_KERN_COUNT = 14
} sttd_kernel;

sttd_status sttd_profile_enable(uint32_t mask);
sttd_status sttd_profile_read(int kernel, int64_t *launches /* host */, double *total_ms /* host */);

/* Device-clock timing, usable inside HIP graphs: while enabled, each launch
 * of a family in `mask` takes the next of max_launches device slots (256 KiB
 * each); thread 0 of every workgroup records its start and end on the 100 MHz
 * device clock (s_memrealtime), and a slot's span runs from the first start to
 * the last end (workgroups beyond the first 12288 of a launch go unrecorded).
 * A captured graph keeps its slots: sttd_clock_reset re-arms the slots handed
 * out so far (call it between replays, outside any capture), and
 * sttd_clock_read sums the spans of one family (microseconds) over the slots
 * stamped since. Enabling with more slots than before reallocates them, which
 * invalidates graphs captured with the old ones. enable/reset/read synchronise
 * the device. */
sttd_status sttd_clock_enable(uint32_t mask, int max_launches);
sttd_status sttd_clock_disable(void);
sttd_status sttd_clock_reset(void);
sttd_status sttd_clock_read(int kernel, int64_t *launches /* host */, double *total_us /* host */);
/* The raw slots in launch order (a timeline): kinds[i] is the family of slot i,
 * start_end[2i], start_end[2i+1] its first start and last end in 100 MHz ticks
 * (~0 and 0 when the launch has not run since the last reset). Copies at most
 * `max` slots; *n receives the number copied. Host buffers. */
sttd_status sttd_clock_spans(int max, int *kinds, uint64_t *start_end, int *n);

#ifdef __cplusplus
}
#endif

#endif /* STTD_H */
