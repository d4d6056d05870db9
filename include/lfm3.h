/*
 * lfm3.h -- C ABI of the MI355X (gfx950) LFM3-1.7B hybrid-decoder forward pass.
 *
 * The library runs the decoder described on the "LFM3-1.7B port" knowledge note (comparison table:
 * 24 layers at width 2048, 13 gated short-conv layers with a 7-tap kernel and a 6-column kept
 * state, 11 GQA attention layers with 16 q / 4 kv heads of 128, six full layers with partial RoPE
 * at theta 1e6 and five sliding layers over 256 tokens with RoPE at theta 1e4, a per-head sigmoid
 * output gate, sandwich RMSNorms with eps 1e-5, a SwiGLU FFN of 7680 and a tied 128000-row head),
 * with MLX-style affine-quantized linears (TensorFold issue #1491, "Checkpoint handling": 4/6/8-bit
 * codes in groups of 64 or 32, bf16 scale and bias per group). Matmul operands, the KV cache and
 * the conv state are fp16; reductions, linear outputs and the residual stream are fp32; the
 * quantized weights are used as stored (exact in decode). It runs as chunked prompt prefill
 * and as batched one-token decode over per-slot streams (TensorFold PR #1508: per-slot conv
 * states, sliding rings and full-attention KV in pool pages; --parallel lanes).
 *
 * Conventions for every call below:
 *  - Memory: the caller allocates every device region (weight blob, workspace, inputs, outputs)
 *    and keeps it alive until lfm3_destroy. The library never allocates device memory.
 *    Pointers named *_dev are device pointers; *_host are host pointers, read during the call only.
 *  - Asynchrony: work is enqueued on the HIP stream given to lfm3_create; results are valid after
 *    that stream is synchronised. Greedy ids stay on the device, so a decode loop needs no host sync.
 *  - Errors: every argument, capacity and slot check runs on the host before anything is enqueued;
 *    on error nothing is enqueued, the state is unchanged, and lfm3_last_error() names the cause.
 *    Two kinds of error are found later. Token ids live on the device, so they are checked by the
 *    embedding kernel: an id outside [0, vocab) embeds as a zero row and raises a device flag that
 *    the next lfm3_synchronize() reports as LFM3_ERR_ARG (the call that enqueued it returned
 *    LFM3_OK). A HIP launch failure (LFM3_ERR_DEVICE) inside lfm3_prefill or lfm3_decode_batch can
 *    leave the slots of that call partly advanced: reset them before using them again.
 *  - Threading: one context per stream; a context is not thread-safe.
 *  - Layouts: row-major. bf16/fp16 are passed as uint16_t bit patterns. Hidden rows are [rows, hidden].
 */
#ifndef LFM3_H
#define LFM3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LFM3_OK = 0,
  LFM3_ERR_ARG = 1,      /* null pointer, bad row count, duplicate slot; token id out of [0, vocab)
                            (reported by lfm3_synchronize)                                           */
  LFM3_ERR_CONFIG = 2,   /* geometry or scheme this build does not run (named in the message)      */
  LFM3_ERR_BLOB = 3,     /* weight blob header: magic, names, shapes, dtypes, byte ranges, size      */
  LFM3_ERR_SLOT = 4,     /* slot index outside [0, max_slots)                                       */
  LFM3_ERR_CAPACITY = 5, /* rows past max_ctx, page pool exhausted, workspace too small              */
  LFM3_ERR_DEVICE = 6    /* not a gfx950 device, or a HIP call failed                               */
} lfm3_status;

enum { LFM3_LAYER_CONV = 0, LFM3_LAYER_FULL = 1, LFM3_LAYER_SLIDING = 2 };
enum { LFM3_MAX_LAYERS = 64, LFM3_MAX_BATCH = 64 };

/*
 * Model and runtime configuration. Every field is explicit; nothing has a default (the
 * "LFM3-1.7B port" note keeps one RoPE dict per layer type; reading a single legacy theta is a
 * known trap on a sibling model's card).
 *   geometry:  n_layers, hidden, ffn, n_q_heads, n_kv_heads, head_dim, vocab, conv_taps, window,
 *              layer_type[i] in {LFM3_LAYER_CONV, _FULL, _SLIDING}
 *   RoPE:      rope_theta_full / rope_pairs_full (1e6, 32 of 64 pairs rotate: partial, zero tail);
 *              rope_theta_sliding / rope_pairs_sliding (1e4, all 64 pairs)
 *   norms:     norm_eps (1e-5)
 *   weights:   bits in {4, 6, 8}, group in {32, 64} for every linear (MLX affine), or bits 16 for
 *              linears stored as bf16 (group ignored); embed_bits / embed_group the same for the
 *              tied embedding and head; has_embedding = 0 runs without embedding and head (rows
 *              enter as hidden states, the output is the final normed hidden state);
 *              ffn_format: LFM3_FFN_AS_LINEARS (w13 and w2 as bits / group say),
 *              LFM3_FFN_NVFP4 (the FFN as e2m1 codes in groups of 16 with e4m3 block scales and an
 *              fp32 tensor scale, weight-only: the static input scale is admitted, not applied --
 *              "TensorFold PR #1508", the layout of the NVFP4 export, whose other linears are
 *              bf16) or LFM3_FFN_FP8_BLOCK (e4m3 codes with one fp32 scale per 128 x 128 block)
 *   runtime:   max_slots streams, max_ctx positions per slot, page_tokens positions per KV page
 *              (16), max_chunk rows per prefill pass, n_pages pages in the full-attention pool
 * This build runs head_dim 128, n_q_heads = 4 * n_kv_heads, conv_taps <= 8, page_tokens 16,
 * hidden (<= 4096) and ffn multiples of 512, max_ctx <= 65536; anything else is refused with
 * LFM3_ERR_CONFIG.
 */
enum { LFM3_FFN_AS_LINEARS = 0, LFM3_FFN_NVFP4 = 1, LFM3_FFN_FP8_BLOCK = 2 };
typedef struct lfm3_config {
  int32_t n_layers, hidden, ffn, n_q_heads, n_kv_heads, head_dim, vocab, conv_taps, window;
  int32_t rope_pairs_full, rope_pairs_sliding;
  int32_t bits, group, embed_bits, embed_group, has_embedding;
  int32_t max_slots, max_ctx, page_tokens, max_chunk, n_pages;
  float norm_eps;
  double rope_theta_full, rope_theta_sliding;
  uint8_t layer_type[LFM3_MAX_LAYERS];
  int32_t ffn_format;
} lfm3_config;

typedef struct lfm3_ctx lfm3_ctx;

/* Sizes the caller must allocate: the exact weight-blob size this config implies (the tensor set
 * and byte ranges of the MLX affine exports, TensorFold issue #1491 "Checkpoint handling"; 594
 * tensors and 973,008,384 data bytes at 4-bit g64 per TensorFold PR #1508's admission commit) and
 * the device workspace (KV pool pages allocated once within a budget, as PR #1508's pool-page
 * commit does; sliding rings, conv states, RoPE tables, activation scratch, a re-tiled copy of
 * every linear's codes and scales for the MFMA paths, and at 6 bits an fp16 copy of the layers'
 * dequantised linears for the prefill GEMM: 2 more bytes per weight). Host only. */
lfm3_status lfm3_query_sizes(const lfm3_config* cfg, size_t* blob_bytes, size_t* workspace_bytes);

/* Admission of a weight blob held in host memory: magic, version, every tensor's name, dtype,
 * shape and byte range against what cfg implies, and the total size (TensorFold #1491: the loader
 * checks names, shapes, dtypes and byte ranges before any kernel runs). Host only; err may be NULL. */
lfm3_status lfm3_validate_blob(const lfm3_config* cfg, const void* blob_host, size_t blob_bytes,
                               char* err, size_t err_len);

/* Create a context (TensorFold issue #1491, "Checkpoint handling": names, shapes, dtypes and byte
 * ranges are admitted before any kernel runs; unsupported schemes are refused by name).
 * blob_dev holds the blob (validated by reading its header back); workspace_dev
 * holds at least workspace_bytes from lfm3_query_sizes. hip_stream is a hipStream_t (NULL = the
 * default stream). Zeroes every slot, uploads the RoPE tables (built in float64, stored fp32) and
 * enqueues the re-tiling of the prefill GEMM weights from the blob on hip_stream (the blob must
 * stay unchanged while the context lives). */
lfm3_status lfm3_create(const lfm3_config* cfg, const void* blob_dev, size_t blob_bytes,
                        void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                        lfm3_ctx** out);

void lfm3_destroy(lfm3_ctx* ctx);

/*
 * Prompt prefill: append n_rows rows to `slot`, starting at its current length, in passes of at
 * most max_chunk rows that carry the conv states, sliding rings and pages across passes ("LFM3-1.7B
 * port", "Chunked prefill"). Exactly one input: tokens_dev int32 [n_rows] (needs has_embedding) or
 * hidden_dev bf16 [n_rows, hidden]. Optional outputs (NULL to skip): logits_last_dev fp32 [vocab]
 * and argmax_last_dev int32 [1] for the last row (needs has_embedding); hidden_out_dev fp32
 * [n_rows, hidden], the final normed hidden state of every row.
 */
lfm3_status lfm3_prefill(lfm3_ctx* ctx, int32_t slot, const int32_t* tokens_dev,
                         const uint16_t* hidden_dev, int32_t n_rows, float* logits_last_dev,
                         int32_t* argmax_last_dev, float* hidden_out_dev);

/*
 * One decode step over several streams in one launch per kernel (TensorFold PR #1508: decode rows
 * of up to eight streams a launch, per-slot conv states, rings and pages; --parallel lanes), for
 * n distinct slots (1 <= n <= min(max_slots, LFM3_MAX_BATCH)): row b appends
 * one position to slots_host[b]. Input: tokens_dev int32 [n] or hidden_dev bf16 [n, hidden].
 * Outputs (NULL to skip): logits_dev fp32 [n, vocab], argmax_dev int32 [n] (greedy id: ties go to
 * the lower id, NaN ranks as -inf), hidden_out_dev fp32 [n, hidden].
 */
lfm3_status lfm3_decode_batch(lfm3_ctx* ctx, int32_t n, const int32_t* slots_host,
                              const int32_t* tokens_dev, const uint16_t* hidden_dev,
                              float* logits_dev, int32_t* argmax_dev, float* hidden_out_dev);

/*
 * Drafted decoding with verify windows ("TensorFold PR #1508": each stream leases one verify window;
 * the short conv runs over each stream's state with every window row's snapshot, and an accepted
 * row's conv state is committed; checked drafted == plain; TensorFold issue #1491, "Validation":
 * partial acceptance). lfm3_verify appends n_rows positions (1 <= n_rows <= min(16, max_chunk)) to
 * `slot` in one prefill pass and returns every row's logits fp32 [n_rows, vocab] and greedy id
 * int32 [n_rows] (either may be NULL, not both): row i scores the token after tokens_dev[i]. The
 * slot then holds an uncommitted window, and until lfm3_commit (or a reset / state load) no other
 * call takes it (LFM3_ERR_ARG). lfm3_commit keeps the first n_accept rows (0 <= n_accept <= n_rows):
 * the slot's length becomes its length before the window + n_accept, its conv states those after
 * row n_accept - 1, and pages past the kept positions go back to the pool. Keys and values of
 * dropped rows stay in the cache but are never read: the next position's are written before any
 * query sees them. Needs has_embedding.
 */
lfm3_status lfm3_verify(lfm3_ctx* ctx, int32_t slot, const int32_t* tokens_dev, int32_t n_rows, float* logits_dev,
                        int32_t* argmax_dev);
lfm3_status lfm3_commit(lfm3_ctx* ctx, int32_t slot, int32_t n_accept);

/*
 * Kept states ("TensorFold PR #1508": a state at `at` is the slot's conv states and its keys and
 * values at positions [0, at), kept in memory allocated once inside the prompt-cache budget so a
 * keep or a restore allocates nothing, and checked resumed == fresh; "LFM3-1.7B port", the
 * checkpoint and rewind paragraph: the conv state must be restored too, else the logits move).
 * A state of a slot holding L positions is: the conv states of every conv layer, the full layers'
 * keys and values of positions [0, L), and the sliding layers' keys and values of the last
 * window - 1 positions (all that the next position sees); its size is a function of L alone.
 * The caller owns the buffer (device memory, 256-byte aligned) and keeps the length.
 */
/* Bytes of a state at `length` positions (0 <= length <= max_ctx). Host only. */
lfm3_status lfm3_state_bytes(const lfm3_ctx* ctx, int32_t length, size_t* bytes);
/* Enqueue a copy of `slot`'s state at its current length into dst_dev (>= lfm3_state_bytes of
 * that length); *length_out (nullable) receives the length. The slot is unchanged. */
lfm3_status lfm3_save_state(lfm3_ctx* ctx, int32_t slot, void* dst_dev, size_t dst_bytes, int32_t* length_out);
/* Make `slot` hold the state in src_dev saved at `length` positions (from any slot of a context of
 * the same geometry): the slot is emptied, pages for `length` positions are leased from the pool
 * (LFM3_ERR_CAPACITY, with nothing changed, if they are not there), the state is copied in and the
 * slot's length set. The next prefill or decode of the slot continues from it. */
lfm3_status lfm3_load_state(lfm3_ctx* ctx, int32_t slot, const void* src_dev, size_t src_bytes, int32_t length);

/* Empty a slot: length 0, conv state zero, its pages back to the pool (TensorFold issue #1491,
 * "Validation": snapshots and reset are among the exactness cases; a reset slot must decode as a
 * fresh one). */
lfm3_status lfm3_reset_slot(lfm3_ctx* ctx, int32_t slot);

/* Synchronise the context's stream and report the device-side argument checks of the calls
 * enqueued since the last synchronize: LFM3_ERR_ARG if a token id outside [0, vocab) reached the
 * embedding (the flag is then cleared), LFM3_ERR_DEVICE if the stream failed, else LFM3_OK. */
lfm3_status lfm3_synchronize(lfm3_ctx* ctx);

/* Current length of a slot (positions held), or -1 for a bad slot. */
int32_t lfm3_slot_length(const lfm3_ctx* ctx, int32_t slot);

/* Free pages in the full-attention pool (a census after resets), or -1 for a NULL ctx. */
int32_t lfm3_free_pages(const lfm3_ctx* ctx);

/* Message of the last failed call on ctx; with ctx NULL, of the last failed lfm3_create or
 * host-only call on this thread. Never NULL. */
const char* lfm3_last_error(const lfm3_ctx* ctx);

/*
 * Debug capture of the residual stream: while set, every later prefill / decode call writes the
 * residual after each layer to dev_buf fp32 [n_layers, max_rows, hidden] (row r of the call at
 * [layer, r, :]; a call may not have more rows than max_rows). dev_buf NULL turns it off. Used by
 * the per-layer rel-L2 parity tests.
 */
lfm3_status lfm3_capture_layers(lfm3_ctx* ctx, float* dev_buf, int32_t max_rows);

/*
 * Run the library's own dequantisation of one stored linear (name as in the blob, without the
 * .q/.scales/.biases suffix) for rows [row0, row0 + n_rows): out_f32_dev [n_rows, K] receives
 * q * scale + bias as computed on the device in fp32 (the embedding's value; the decode GEMV never
 * forms it, using scale * sum(x q) + bias * sum(x) with exact q) and out_f16_dev [n_rows, K] its
 * round-to-nearest-even fp16 (the value the prefill GEMM stages in LDS). Either output may be
 * NULL. For the bit-exact dequant parity test.
 */
lfm3_status lfm3_dequant_rows(lfm3_ctx* ctx, const char* name, int32_t row0, int32_t n_rows,
                              float* out_f32_dev, uint16_t* out_f16_dev);

/*
 * One stored linear (name without the .q/.scales/.biases suffix) applied to caller rows, for
 * kernel-level parity: y_dev fp32 [rows, N] = x_dev fp16 [rows, K] times the dequantised weight,
 * through the decode dequant-GEMV (path 0, rows in [1, 8], exact weights), the prefill MFMA GEMM
 * (path 1, weights rounded to fp16; at 6 bits read from the fp16 copy), the same GEMM always
 * dequantising the codes in its K loop (path 6; bitwise the same result as path 1) or the decode MFMA GEMM of 3+ rows
 * (path 4, rows in [1, 64], weights rounded to fp16). Paths 2 (GEMV), 3 (GEMM) and 5 (decode MFMA)
 * apply the SwiGLU epilogue of a fused [gate | up] weight instead: y_dev then receives fp16
 * [rows, N/2] = silu(gate) * up. The embedding (tied head) has only path 0.
 */
lfm3_status lfm3_linear(lfm3_ctx* ctx, const char* name, int32_t path, const uint16_t* x_dev,
                        int32_t rows, float* y_dev);

/*
 * Kernel-level hook of one attention layer's core on caller buffers, for parity at the served
 * shapes: the per-head q/k RMSNorm + RoPE of the rows' own queries and keys, the store of their
 * keys and values into the caller's cache, attention over every visible key, and the sigmoid head
 * gate, through the same launches a prefill pass or decode step makes ("LFM3-1.7B port":
 * comparison table rows 2-4, the sliding-window mask section and "partial_rotary_factor";
 * "TensorFold PR #1508": KV in 16-token pool pages under a per-slot page table, four query heads
 * a KV head, decode rows of several streams in one launch).
 *
 *   sliding       0: a full layer (RoPE theta_full on rope_pairs_full pairs; keys j <= p; the cache
 *                 is paged); 1: a sliding layer (theta_sliding, rope_pairs_sliding; keys with
 *                 0 <= p - j < window; the cache is a per-slot ring).
 *   decode        1: n_rows rows, row b appends position pos_host[b] to slot slots_host[b]
 *                 (distinct slots, 1 <= n_rows <= min(max_slots, LFM3_MAX_BATCH)): the split-K
 *                 decode kernel and its merge. 0: one prefill pass, n_rows consecutive positions
 *                 from pos_host[0] of slot slots_host[0] (1 <= n_rows <= max(max_chunk, max_slots)):
 *                 the q/k norm + RoPE + KV-store kernel, then the flash prefill kernel.
 *   qkvg_dev      fp32 [n_rows, ld]: the raw qkvg linear output of each row, q (n_q_heads x 128) |
 *                 k (n_kv_heads x 128) | v (n_kv_heads x 128) | g (n_q_heads), ld >= that width.
 *   q_norm_dev, k_norm_dev   bf16 [128]: the per-head RMSNorm weights.
 *   k_cache_dev, v_cache_dev fp16 caches, caller-owned; positions before each row's own hold the
 *                 keys (after norm + RoPE) and values of the slot's history. Full: [n_pool_pages,
 *                 n_kv_heads, 16, 128], position p of slot s in page page_table_dev[s * max_pages +
 *                 p / 16], row p % 16. Sliding: [n_slots, n_kv_heads, ring_rows, 128], position p at
 *                 ring row p % ring_rows. The call writes each row's own key and value there; it
 *                 reads no cache row that holds no visible key (such rows may hold anything).
 *   page_table_dev int32 [n_slots, max_pages] (full layers only; every page covering positions
 *                 0 .. the last row's position of a used slot in [0, n_pool_pages)).
 *   out_dev       fp16 [n_rows, n_q_heads * 128]: sigmoid(g_h) * attention output of head h.
 * Every position must be < max_ctx (the context's RoPE tables). Sliding rings need ring_rows >=
 * window in decode and >= window + n_rows - 1 in prefill (a pass's own keys must not overwrite
 * keys its first row still sees); full layers need max_pages <= 8192. Split partials and the prefill's rotated queries use the
 * context's workspace, so one call at a time per context. The full layer's page table is copied
 * to the host and checked before anything is enqueued (this synchronises the device); any check
 * failing returns LFM3_ERR_ARG with nothing enqueued.
 */
typedef struct lfm3_attn_io {
  int32_t sliding, decode, n_rows;
  const int32_t* slots_host;
  const int32_t* pos_host;
  const float* qkvg_dev;
  int32_t ld;
  const uint16_t* q_norm_dev;
  const uint16_t* k_norm_dev;
  uint16_t* k_cache_dev;
  uint16_t* v_cache_dev;
  const int32_t* page_table_dev;
  int32_t max_pages, n_pool_pages, n_slots, ring_rows;
  uint16_t* out_dev;
} lfm3_attn_io;
lfm3_status lfm3_attention(lfm3_ctx* ctx, const lfm3_attn_io* io);

/*
 * lfm3_attention in decode mode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the split partials in a fixed device array of the library (4.4 MB per GPU, kept
 * until the process ends) instead of the context's workspace, and no device-to-host copy: the
 * page table of a full layer is checked from page_table_host, a host copy of page_table_dev with
 * the same layout (NULL for sliding layers). Takes decode rows only, 1 <= n_rows <= 8; more
 * rows return LFM3_ERR_CAPACITY, other argument errors LFM3_ERR_ARG, with nothing enqueued. The
 * array is shared by every call on a GPU: calls that overlap on one GPU (several contexts or
 * streams at once) race; calls in one stream's order do not.
 */
lfm3_status lfm3_attention_noalloc(lfm3_ctx* ctx, const lfm3_attn_io* io, const int32_t* page_table_host);

/*
 * Kernel-family timing for roofline figures. lfm3_profile(ctx, 1) starts recording: every later
 * launch is tagged with its family and the algorithmic bytes and flops it implies (weights +
 * activations read and written; 2*M*N*K for a linear; 4*128*heads per visible key for
 * attention), and each run of consecutive launches of one family is bracketed by one pair of HIP
 * events on the context's stream (so the time is back-to-back kernel execution, with no event
 * between two kernels of a run). lfm3_profile(ctx, 0) stops; either call drops earlier records.
 * lfm3_profile_read synchronises the stream and returns, for one family, the summed event time
 * (ms), the launch count and the summed bytes and flops. Any output may be NULL. Recording adds
 * an event pair per run, so throughput is measured with recording off.
 */
enum {
  LFM3_PROF_GEMV = 0,          /* decode dequant-GEMV (linears and the tied head)   */
  LFM3_PROF_GEMM = 1,          /* prefill dequant-to-LDS MFMA GEMM                  */
  LFM3_PROF_ATTN_DECODE = 2,   /* split-K decode attention + merge                  */
  LFM3_PROF_ATTN_PREFILL = 3,  /* flash prefill attention                           */
  LFM3_PROF_CONV = 4,          /* gated short conv                                  */
  LFM3_PROF_NORM = 5,          /* residual + RMSNorm                                */
  LFM3_PROF_OTHER = 6,         /* q/k norm + RoPE + KV store, embedding, argmax, page table */
  LFM3_PROF_KINDS = 7
};
lfm3_status lfm3_profile(lfm3_ctx* ctx, int32_t enable);
lfm3_status lfm3_profile_read(lfm3_ctx* ctx, int32_t kind, double* total_ms, int64_t* launches,
                              double* bytes, double* flops);

#ifdef __cplusplus
}
#endif

#endif /* LFM3_H */
