/*
 * cbd.h - C ABI of libcbd.so: continuous-batching transformer decode on one
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (as defined on the page "Continuous Decode Batching - the
 * transformer capture"):
 *  - decode_step_batch: section "decode_step_batch - paint-by-numbers" and
 *    section "1. Native station: per-sequence KV + a batched decode step".
 *    B live sequences take one step together. Every weight matrix is read
 *    from HBM once for the whole batch (the page's "throughput law":
 *    sharedCost = w + L*a instead of L*(w + a)); each row applies RoPE at its
 *    own position t_s, appends its K/V to its own slab at t_s, attends to
 *    [0..=t_s] of that slab only, and gets one row of lm_head logits; then
 *    its length becomes t_s + 1.
 *  - prefill_segmented: section "REVISED ... forward_batch_segmented". K
 *    prompts packed into one pass; every projection runs once over all
 *    tokens; attention is block-diagonal causal (a token attends only to
 *    earlier tokens of its own sequence); positions continue from the
 *    sequence's length (0 for a fresh slab), so a prompt can be admitted in
 *    chunks between decode steps (page "Batching", section 4.2). Returns the
 *    logits of each segment's last token only.
 *  - kvslab_alloc / kvslab_free: section "1. Native station": an N-slot KV
 *    arena keyed by sequence id; admission = fresh slab at length 0, EOS =
 *    drop the slab; capacity is bounded and the caller queues what does
 *    not fit (section "2. JS scheduler", "Backpressure").
 *  - greedy_argmax / sample_top_p: the token of each logits row, greedy or
 *    seeded temperature / top-p (page "Batching", later revision, section
 *    4.4 and section 8).
 *  - kvslab_fork: page "Batching", section 6, item 3: a sequence that
 *    starts from another's first positions shares that prefix's K/V blocks
 *    (copy-on-write of the block where the prefix ends).
 *  - kv_format (cbd_model_config): slabs hold bf16 K/V, or affine 8-bit /
 *    4-bit codes with a (scale, bias) pair per group of 64 dims (page
 *    "Batching", sections 4.3 and 6: quantized caches as packed values,
 *    scales and biases).
 *
 * Model body (the pages do not spell it out; plainest Llama/Mistral reading):
 * RMSNorm (y = x / sqrt(mean(x^2) + eps) * g), GQA attention with rotate-half
 * RoPE (angle t * theta^(-2i/Dh)), scale 1/sqrt(Dh), SwiGLU FFN
 * (W_down(silu(W_gate x) * W_up x)), final RMSNorm, untied lm_head.
 *
 * Numerics: residual stream, softmax and every accumulation in fp32; weight
 * operands of matrix products in bf16 (or int4-affine dequantized to bf16
 * in registers), activation operands as a bf16 pair hi = bf16(x),
 * lo = bf16(x - hi) (about 16 significant bits); K/V stored in the slabs as
 * bf16 (round to nearest even), or quantized from that bf16 value; logits
 * fp32.
 *
 * Memory ownership: the caller owns every device buffer it passes (weights,
 * KV arena, token and logit buffers) and every stream. The library
 * allocates its own fixed-size device workspace once, in cbd_create, and
 * frees it in cbd_destroy; no entry point allocates device memory after
 * that. Pointers named *_dev are device pointers; all others are host.
 *
 * Streams: every device operation is enqueued on the given stream (NULL =
 * the null stream) and returns without waiting. All calls on one context
 * must be serialized on one stream: the context's workspace is shared.
 *
 * Errors: every call returns a cbd_status. Arguments are validated on the
 * host before anything is enqueued; when a call fails, no slab length and
 * no slab content changes. cbd_last_error() gives a message for the last
 * failure on the calling thread. Asynchronous device faults are reported by
 * the HIP runtime on the next synchronizing call (CBD_E_HIP).
 */
#ifndef CBD_H
#define CBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cbd_ctx cbd_ctx;
typedef void* cbd_stream; /* a hipStream_t */

typedef enum {
  CBD_OK = 0,
  CBD_E_INVAL = -1,    /* bad argument (null pointer, size out of range, duplicate id, ...) */
  CBD_E_NOSPACE = -2,  /* arena cannot hold the slab now: queue the request and retry later */
  CBD_E_CAPACITY = -3, /* the slab's capacity (or the RoPE table) would be exceeded */
  CBD_E_BADSEQ = -4,   /* unknown or freed sequence id */
  CBD_E_HIP = -5,      /* a HIP runtime call failed */
  CBD_E_NODEVICE = -6, /* context was created host-only: bookkeeping works, device work does not */
  CBD_E_UNSUPPORTED = -7 /* the call is not available for this context's K/V storage format */
} cbd_status;

enum { CBD_WEIGHTS_BF16 = 0, CBD_WEIGHTS_INT4 = 1 };

/*
 * K/V storage of the slabs (mlx-bun "Batching" design note, section 4.3: a quantized cache is held
 * as (packed values, scales, biases); section 6 "KV memory model": quantized K/V multiplies the
 * arena's capacity).
 *  CBD_KV_BF16:    every K/V element is stored as bf16 (rounded to nearest even).
 *  CBD_KV_AFFINE8: each group of 64 consecutive dims of one head vector is stored as 8-bit codes
 *                  with a float32 (scale, bias) pair: bias = the group's minimum, scale = (maximum -
 *                  bias) / 255, code = (x - bias) / scale rounded half to even and clamped to 0..255
 *                  (decided in float32; code 0 when scale = 0), where x is the element's bf16 value;
 *                  attention reads scale * code + bias. 144 bytes per token, layer and KV head at
 *                  head_dim 128 (bf16: 256). decode_step_batch, prefill_segmented (whose tokens
 *                  attend to the stored, quantized keys of their own segment) and kvslab_append
 *                  quantize on append; kvslab_read returns CBD_E_UNSUPPORTED (kvslab_read_q8 reads
 *                  the stored form).
 *  CBD_KV_AFFINE4: the same with 4-bit codes (maximum code 15, scale = (maximum - bias) / 15), two
 *                  per byte: 80 bytes per token, layer and KV head at head_dim 128.
 */
enum { CBD_KV_BF16 = 0, CBD_KV_AFFINE8 = 1, CBD_KV_AFFINE4 = 2 };

typedef struct {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;      /* query heads */
  int32_t n_kv_heads;   /* n_heads must be a multiple of n_kv_heads (GQA) */
  int32_t head_dim;     /* 64 or 128 */
  int32_t ffn_dim;
  int32_t vocab;        /* multiple of 64 */
  float rms_eps;
  float rope_theta;
  int32_t weight_format; /* CBD_WEIGHTS_BF16 or CBD_WEIGHTS_INT4 */
  int32_t max_position;  /* length of the RoPE table: no slab may grow beyond it */
  int32_t kv_format;     /* CBD_KV_BF16 (0), CBD_KV_AFFINE8 (1) or CBD_KV_AFFINE4 (2) */
} cbd_model_config;

/*
 * One weight matrix W [N, K] (N outputs, K inputs; y = W x), in the
 * library's streaming layout (each weight is read once per step, so the
 * layout is chosen for sequential HBM reads):
 *  bf16 format: data = bf16 as written by cbd_pack_bf16 from a row-major
 *  [N, K] matrix; aux unused.
 *  int4 format (4-bit affine, groups of 64 consecutive inputs of one row,
 *  w = scale * code + bias with codes 0..15): data = packed codes and aux =
 *  bf16 (scale, bias) pairs, both as written by cbd_pack_int4.
 *  N must be a multiple of 16; K a multiple of 32 (bf16) or 128 (int4).
 */
typedef struct {
  const void* data;
  const void* aux;
} cbd_matrix;

typedef struct {
  const void* attn_norm; /* bf16 [d_model] */
  cbd_matrix wq;         /* [n_heads*head_dim, d_model] */
  cbd_matrix wk;         /* [n_kv_heads*head_dim, d_model] */
  cbd_matrix wv;         /* [n_kv_heads*head_dim, d_model] */
  cbd_matrix wo;         /* [d_model, n_heads*head_dim] */
  const void* ffn_norm;  /* bf16 [d_model] */
  cbd_matrix w_gate;     /* [ffn_dim, d_model] */
  cbd_matrix w_up;       /* [ffn_dim, d_model] */
  cbd_matrix w_down;     /* [d_model, ffn_dim] */
} cbd_layer_weights;

typedef struct {
  const void* embed;                /* bf16 [vocab, d_model]; gathered, never streamed */
  const void* final_norm;           /* bf16 [d_model] */
  cbd_matrix lm_head;               /* [vocab, d_model] */
  const cbd_layer_weights* layers;  /* host array [n_layers]; copied by cbd_create */
} cbd_weights;

typedef struct {
  int32_t max_batch;          /* rows per decode_step_batch call, 1..64 */
  int32_t max_prefill_tokens; /* sum of segment lengths per prefill_segmented call */
  int32_t max_segments;       /* segments per prefill_segmented call, 1..64 */
  int32_t host_only;          /* nonzero: no device memory, no kernels (host bookkeeping tests) */
} cbd_limits;

typedef struct {
  int64_t live_seqs;
  int64_t arena_bytes;
  int64_t arena_bytes_used;
  int64_t decode_steps;
  int64_t decode_rows;
  int64_t prefill_calls;
  int64_t prefill_tokens;
} cbd_stats_t;

/* Bytes of K and V one token occupies in a slab, over all layers: n_layers * 2 * n_kv_heads *
 * head_dim * 2 for bf16 slabs, n_layers * 2 * n_kv_heads * (head_dim * b / 8 + head_dim / 64 * 8)
 * for affine slabs of b-bit codes (b = 8 or 4). */
size_t cbd_kv_bytes_per_token(const cbd_model_config* cfg);

/* Tokens per arena granule: slab capacities are rounded up to a multiple. */
int32_t cbd_slab_granule_tokens(void);

/*
 * Create a context. Weights are referenced, not copied: they must stay
 * valid until cbd_destroy; every weight pointer (matrices, int4 scale/bias
 * pairs, norm gains, embedding) must be 16-byte aligned (CBD_E_INVAL). kv_arena_dev (arena_bytes long, 256-byte
 * aligned) is caller-owned device memory that the library carves into
 * per-sequence slabs; it is cleared here and must not be written by the
 * caller while the context lives (slab contents are read and written only
 * through kvslab_append / kvslab_read and the step calls; their internal
 * layout is private). Allocates the device workspace (sized by limits) and
 * the RoPE table (built on the host in double precision, stored as fp32).
 * Returns CBD_E_INVAL on inconsistent shapes, CBD_E_HIP if the workspace
 * cannot be allocated. With limits->host_only the weight and arena pointers
 * may be NULL (arena_bytes still sets the arena size).
 */
cbd_status cbd_create(const cbd_model_config* cfg, const cbd_weights* weights, const cbd_limits* limits,
                      void* kv_arena_dev, size_t arena_bytes, cbd_ctx** out);

/* Release the workspace (waits for the device). The arena and weights stay the caller's. */
cbd_status cbd_destroy(cbd_ctx* ctx);

/* Message for the last failed call on this thread ("" if none). Valid until the next call. */
const char* cbd_last_error(void);

/* Totals since cbd_create. */
cbd_status cbd_stats(const cbd_ctx* ctx, cbd_stats_t* out);

/*
 * Admit a sequence: reserve a slab of capacity_tokens (rounded up to the
 * granule) at length 0. Ids are small non-negative integers, reused after
 * kvslab_free. CBD_E_NOSPACE if no contiguous run of the arena is free now;
 * CBD_E_CAPACITY if the capacity exceeds max_position or the whole arena.
 */
cbd_status kvslab_alloc(cbd_ctx* ctx, int32_t capacity_tokens, int32_t* seq_id_out);

/* Retire a sequence (EOS or length limit): its slab returns to the arena. A sequence that live forks
 * still read (kvslab_fork) keeps its memory until the last of them is freed; its id is retired at once. */
cbd_status kvslab_free(cbd_ctx* ctx, int32_t seq_id);

/*
 * Start a sequence from the first prefix_len positions of a live sequence (mlx-bun "Batching" design
 * note, section 6 "KV memory model", item 3: paged K/V with block-level copy-on-write prefix
 * sharing). The fork's length is prefix_len; its capacity is capacity_tokens (> prefix_len, counting
 * the prefix). Whole blocks of 32 keys of the prefix are not copied: the fork reads them from the
 * parent's slab in every later call, so they occupy the arena once however many forks share them.
 * The block that holds the prefix's last keys, when prefix_len is not a multiple of 32, is copied
 * into the fork (on `stream`, from the parent's slab as it stands; positions below prefix_len never
 * change, so the parent may keep decoding). The fork's own part takes ceil((capacity_tokens -
 * floor(prefix_len / 32) * 32) / granule) granules. The parent must not itself be a fork
 * (CBD_E_INVAL); CBD_E_NOSPACE / CBD_E_CAPACITY as kvslab_alloc. A host-only context keeps the
 * bookkeeping and copies nothing.
 */
cbd_status kvslab_fork(cbd_ctx* ctx, int32_t parent_seq_id, int32_t prefix_len, int32_t capacity_tokens,
                       int32_t* seq_id_out, cbd_stream stream);

/* Current length t_s (tokens held) and capacity of a live slab. */
cbd_status kvslab_len(const cbd_ctx* ctx, int32_t seq_id, int32_t* len_out);
cbd_status kvslab_capacity(const cbd_ctx* ctx, int32_t seq_id, int32_t* cap_out);

/*
 * Append n_tokens of given K and V to a slab at positions [len, len+n):
 * k_dev, v_dev are bf16 [n_layers, n_tokens, n_kv_heads, head_dim]
 * (K already rotated to its position). Used to seed long histories and to
 * re-inject saved state. An affine 8-bit slab stores them quantized (per
 * token, head and group of 64 dims, as CBD_KV_AFFINE8 states). CBD_E_CAPACITY
 * if len + n_tokens > capacity.
 */
cbd_status kvslab_append(cbd_ctx* ctx, int32_t seq_id, int32_t n_tokens, const void* k_dev,
                         const void* v_dev, cbd_stream stream);

/*
 * Copy positions [start, start+n) of a slab out to k_out_dev, v_out_dev in the
 * layout kvslab_append takes. CBD_E_CAPACITY if start + n > len.
 */
cbd_status kvslab_read(const cbd_ctx* ctx, int32_t seq_id, int32_t start, int32_t n_tokens,
                       void* k_out_dev, void* v_out_dev, cbd_stream stream);

/*
 * Read tokens [start, start + n) of an affine slab (8- or 4-bit codes) in its stored form:
 *  codes_out_dev  device uint8 [L, n, 2, n_kv_heads, head_dim] (index 2: 0 = K, 1 = V), one code
 *                 per byte
 *  sb_out_dev     device float32 [L, n, 2, n_kv_heads, head_dim / 64, 2] (scale, bias)
 * Both 16-byte aligned, caller-owned. CBD_E_UNSUPPORTED on a bf16 context, CBD_E_CAPACITY if
 * start + n > len. For tests and for moving a quantized history out of the arena.
 */
cbd_status kvslab_read_q8(const cbd_ctx* ctx, int32_t seq_id, int32_t start, int32_t n_tokens, void* codes_out_dev,
                          void* sb_out_dev, cbd_stream stream);

/*
 * One batched decode step over B distinct live sequences.
 *  seq_ids          host int32 [B]
 *  last_tokens_dev  device int32 [B]: the token each row feeds (ids outside
 *                   [0, vocab) are clamped; they stay on the device so the
 *                   previous step's argmax can feed this one directly)
 *  logits_dev       device fp32 [B, vocab], written
 *  next_tokens_dev  device int32 [B] or NULL: greedy argmax of each logits
 *                   row (lowest id among equal maxima)
 * Row i uses t = kvslab_len(seq_ids[i]) captured once on the host, writes
 * its K/V at t, attends [0..=t], and its length becomes t + 1.
 * B = 0 is a no-op. CBD_E_INVAL: B > max_batch, duplicate ids, null
 * pointers; CBD_E_BADSEQ: unknown id; CBD_E_CAPACITY: a slab is full.
 */
cbd_status decode_step_batch(cbd_ctx* ctx, const int32_t* seq_ids, int32_t B, const int32_t* last_tokens_dev,
                             float* logits_dev, int32_t* next_tokens_dev, cbd_stream stream);

/*
 * Segmented prefill of K distinct live sequences.
 *  seq_ids     host int32 [K]
 *  seg_lens    host int32 [K], each >= 1
 *  tokens_dev  device int32 [sum(seg_lens)]: the segments back to back
 *  last_logits_dev  device fp32 [K, vocab]: logits of each segment's last token
 *  next_tokens_dev  device int32 [K] or NULL: their greedy argmax
 * Segment s continues its sequence: with t = kvslab_len(seq_ids[s]) before the
 * call (0 for a fresh slab), its tokens take positions t..t+len_s-1, attend to
 * the sequence's keys 0..own position (earlier chunks and decoded tokens
 * included, never another sequence's), are written to the slab there, and the
 * length becomes t + len_s. A long prompt can so be admitted in chunks with
 * decode steps in between (page "Batching", section 4.2: joiner prefill one
 * chunk of at most 2048 tokens per loop iteration, one decode step between
 * chunks). K = 0 is a no-op. CBD_E_INVAL: zero-length segment, duplicate id,
 * K > max_segments, or the total above max_prefill_tokens; CBD_E_CAPACITY:
 * t + len_s above the slab's capacity or max_position.
 */
cbd_status prefill_segmented(cbd_ctx* ctx, const int32_t* seq_ids, const int32_t* seg_lens, int32_t K,
                             const int32_t* tokens_dev, float* last_logits_dev, int32_t* next_tokens_dev,
                             cbd_stream stream);

/*
 * Greedy selection over rows of logits (page "Batching", later revision,
 * section 8: the lowest vocabulary id wins among tied scores).
 * logits_dev fp32 [rows, vocab] -> tokens_dev int32 [rows]. rows <= 64.
 */
cbd_status greedy_argmax(cbd_ctx* ctx, const float* logits_dev, int32_t rows, int32_t* tokens_dev,
                         cbd_stream stream);

/*
 * greedy_argmax without a context and without allocating: for callers that
 * cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid it). The same selection (lowest id among the
 * maxima of each row; token 0 for a row of NaNs) and the same kernel.
 *  logits_dev  device fp32 [rows, vocab], 16-byte aligned (caller-owned)
 *  rows        0..64 (0: no-op); more rows fail with CBD_E_INVAL
 *  vocab       a multiple of 4 in 4..2^30
 *  tokens_dev  device int32 [rows] (caller-owned), written on the stream
 * The kernel's workspace (per-row partial maxima and arrival counters, 33 KB)
 * is a static device array of the library: one copy per GPU, held until the
 * process ends; the first call on a device looks up its address. Every call
 * on one GPU shares that GPU's copy: calls that overlap on one GPU (several
 * streams or threads at once) race and must be serialized by the caller.
 * Calls no hipMalloc/hipFree and enqueues no memset (two kernels on the
 * stream). CBD_E_HIP: no current device or a failed launch.
 */
cbd_status cbd_greedy_argmax_noalloc(const float* logits_dev, int32_t rows, int32_t vocab, int32_t* tokens_dev,
                                     cbd_stream stream);

/*
 * Seeded per-row sampling over rows of logits (page "Batching", later
 * revision, section 4.4 "The decode step": a row's random draw is selected by
 * its request's seed and local sample index, independently of the other rows;
 * temperature 0 is greedy selection with the greedy tie rule).
 *  logits_dev    device fp32 [rows, vocab] (the context's vocab, a multiple of
 *                4; 16-byte aligned). NaN logits weigh nothing.
 *  temperature   host fp32 [rows]: 0 = greedy (lowest id among maxima); > 0
 *                divides the logits before the softmax
 *  top_p         host fp32 [rows] in (0, 1]: the nucleus is the shortest prefix
 *                of the tokens ordered by probability (highest first, equal
 *                probabilities by lower id) whose mass reaches top_p
 *  seeds, sample_index  host uint64 [rows]: the draw u in [0, 1) is the 24
 *                high bits of word 0 of Philox4x64-10 (Salmon et al., SC 2011)
 *                with key (seed, 0) and counter (sample_index, 0, 0, 0), over 2^24
 *  tokens_dev    device int32 [rows], written: the first token of the nucleus
 *                order whose running mass exceeds u times the nucleus mass
 * Probabilities are taken in fixed point, e^(z - max z) in units of 2^-40 with
 * z = logit / temperature; every selection after that is integer arithmetic,
 * so the result does not depend on summation order. Each row is cut into 32
 * chunks of consecutive ids, one workgroup each, over nine launches; the
 * context's workspace holds the weights and the chunks' histograms.
 * rows = 0 is a no-op. CBD_E_INVAL: rows outside 0..64, null or unaligned
 * pointers, a temperature negative or not finite, top_p outside (0, 1], a
 * vocab that is not a multiple of 4.
 */
cbd_status sample_top_p(cbd_ctx* ctx, const float* logits_dev, int32_t rows, const float* temperature,
                        const float* top_p, const uint64_t* seeds, const uint64_t* sample_index,
                        int32_t* tokens_dev, cbd_stream stream);

/*
 * The batched weight-streaming product alone (the page's batched matvec
 * that shares one weight read across all lanes):
 * y_dev[b, n] = sum_k W[n, k] * x_dev[b, k] for b < rows.
 *  x_dev  fp32 [rows, K] row-major (carried internally as two bf16 planes,
 *         hi = bf16(x) and lo = bf16(x - hi));  y_dev fp32 [rows, N].
 * rows 1..64; N a multiple of 64; K a multiple of 256 (bf16 weights) or 512
 * (int4) and at most max(d_model, ffn_dim). Uses the context's weight
 * format. splits selects how the launch is cut (0 = the library's choice):
 * splits > 0: 4-wave workgroups share staged activations and K is divided
 * over `splits` workgroups (it must divide K into multiples of 128);
 * splits = -4, -8 or -16: each workgroup owns 16 weight rows (bf16; 32 for
 * int4) and divides K over that many waves, each wave taking at least two
 * stages of 32 (int4: 128) inputs; bf16 rows <= 64 (<= 8 with -16), int4
 * rows <= 16 (<= 8 with more than 4 waves); CBD_E_INVAL otherwise. Exposed
 * for kernel-level parity tests and bandwidth measurements.
 */
cbd_status cbd_linear(cbd_ctx* ctx, const cbd_matrix* w, int32_t N, int32_t K, const float* x_dev, int32_t rows,
                      float* y_dev, int32_t splits, cbd_stream stream);

/*
 * Pack a row-major bf16 matrix [N, K] (device) into the streaming layout
 * (device, a different buffer of the same size), enqueued on `stream`.
 * Layout: fragments of 16 rows x 32 inputs, 1 KB each; fragment (t, f)
 * (rows 16t.., inputs 32f..) is the (t * K/32 + f)-th; inside it, the 16
 * bytes at offset 16*l hold row 16t + l%16, inputs 32f + 8*(l/16) .. +7.
 * N % 16 == 0, K % 32 == 0.
 */
cbd_status cbd_pack_bf16(const void* src_dev, int64_t N, int64_t K, void* dst_dev, cbd_stream stream);

/*
 * Pack a 4-bit affine matrix into the int4 streaming layout (host memory).
 *  codes   uint8 [N, K], values 0..15 (w = scale * code + bias)
 *  scale, bias  bf16 bits [N, K/64]
 *  packed_out   uint32 [N*K/8]
 *  aux_out      bf16 bits [K/64, N, 2]: (scale, bias) pairs, group-major
 * Packed layout: blocks of 16 rows x 128 inputs, 1 KB each; block (t, b)
 * is the (t * K/128 + b)-th. Inside it, the 4 words at offset 16*l belong
 * to row 16t + r with r = l%16 and g = l/16: word j (0..3) holds the 8
 * codes of inputs 128b + 32*j + 8*g + e, e = 0..7, with input e in nibble
 * (e/2) + 4*(e%2). K % 128 == 0, N % 16 == 0.
 */
cbd_status cbd_pack_int4(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int64_t N,
                         int64_t K, uint32_t* packed_out, uint16_t* aux_out);

/*
 * Per-kernel timing with HIP events (a tracing aid, the counterpart of the
 * per-step trace of page "Batching", section 4.4, "Housekeeping"). Between cbd_profile_begin and
 * cbd_profile_end every launch of a selected kind is bracketed by two
 * events recorded on the launch's own stream. cbd_profile_end waits for the
 * last event and returns, per kind, the launch count, the summed
 * event-to-event milliseconds, and the summed algorithmic bytes and flops
 * of those launches (counted from shapes: weights + activations read +
 * outputs written; K/V bytes read for attention). kind_mask is a bit mask
 * of (1 << cbd_kernel_kind). every >= 1 times one selected launch in
 * `every` (counted over all selected kinds in launch order; 1 = all of
 * them): each timed launch costs the stream a few microseconds of event
 * handling, so sampling keeps a timed run close to an untimed one.
 * max_launches bounds the launches recorded; later ones are not timed.
 * Event handles are created in cbd_profile_begin. CBD_E_INVAL: null
 * context, max_launches outside 0..2^22 or every < 1.
 */
typedef enum {
  CBD_KERNEL_EMBED = 0,
  CBD_KERNEL_NORM = 1,
  CBD_KERNEL_QKV = 2,
  CBD_KERNEL_ROPE_APPEND = 3,  /* prefill only: decode rotates and appends inside attention */
  CBD_KERNEL_ATTENTION = 4,
  CBD_KERNEL_ATTN_COMBINE = 5, /* reserved: splits are merged inside the attention kernel */
  CBD_KERNEL_O_PROJ = 6,
  CBD_KERNEL_GATE_UP = 7,
  CBD_KERNEL_DOWN = 8,
  CBD_KERNEL_LM_HEAD = 9,
  CBD_KERNEL_ARGMAX = 10,
  CBD_KERNEL_SAMPLE = 11,
  CBD_KERNEL_KINDS = 12
} cbd_kernel_kind;

typedef struct {
  int64_t launches;
  double total_ms;
  double bytes;
  double flops;
} cbd_kernel_time;

cbd_status cbd_profile_begin(cbd_ctx* ctx, uint32_t kind_mask, int32_t max_launches, int32_t every);
cbd_status cbd_profile_end(cbd_ctx* ctx, cbd_kernel_time* out /* [CBD_KERNEL_KINDS] */);

#ifdef __cplusplus
}
#endif
#endif /* CBD_H */
