/*
 * qd.h -- C ABI of the int8 weight-only Qwen3-family decoder step for AMD MI355X (gfx950).
 *
 * The library runs the forward step of a Qwen3-family decoder whose projection
 * weights are stored as int8 with one fp32 scale per output row: prompt token ids
 * in, greedily generated token ids out.  It has three workloads: prefill over the
 * whole prompt, single-stream decode (one token per step) and batched decode
 * (B sequences per step, weights swept once per step).  Sources:
 *   - "Model-agnostic LLM inference", section "Supported models": the decoder
 *     family (grouped-query attention, RMSNorm on Q and K, RoPE, SiLU-gated
 *     feed-forward, tied embeddings, no attention bias) and its gates.
 *   - same page, section "The quantized load cache": int8 weights with per-row
 *     scales; section "Notes": greedy arg-max by default, one call runs prefill
 *     then decode up to max_new_tokens or end-of-text; section "Long context":
 *     context sizing and the 65,536-token ceiling; section "Errors": named
 *     error codes, every problem named before any GPU work.
 *   - "LLM inference overview", sections "Results" and "Workload
 *     characteristics": prefill fills the KV cache, decode sweeps all weights per
 *     token, batched decode sweeps them once per step for all B sequences.
 *
 * Precision contract (the pages leave it open; this library fixes it):
 * symmetric per-output-channel int8 codes in [-127, 127] with fp32 scales
 * (scale = absmax / 127, code = round-half-even(w / scale), IEEE fp32 division),
 * bf16 activations rounded at every tensor the model produces, fp32 accumulation,
 * fp32 RMSNorm and softmax, a bf16 KV cache and fp32 logits.
 *
 * Memory ownership: the library never allocates device memory.  The caller
 * allocates three device buffers whose sizes qd_query_sizes() returns (weights,
 * KV cache, workspace) and keeps them alive until qd_free().  A qd_model handle
 * owns host memory and HIP graph objects only.  Every call that takes a stream
 * enqueues its work on that stream and returns without waiting, except where a
 * comment says otherwise.  A handle must be used from one host thread at a time.
 *
 * Errors: every entry point returns a qd_status.  On failure nothing has been
 * enqueued unless the code is QD_ERR_DEVICE, and qd_last_error() returns a
 * message (thread-local, valid until the next call on the same thread) that names
 * every problem found.
 */
#ifndef QD_H
#define QD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* qd_stream;  /* a hipStream_t; NULL is the default stream */

typedef enum {
  QD_OK = 0,
  /* The shape is outside the supported family or its gates ("Model-agnostic LLM
   * inference", sections "Supported models" and "Errors"). */
  QD_ERR_UNSUPPORTED_ARCH = 1,
  /* Empty or out-of-range token ids, max_new_tokens < 1, a batch or context
   * larger than the model was loaded for ("Errors", invalid_arguments). */
  QD_ERR_INVALID_ARGUMENTS = 2,
  /* A context length above 65,536 tokens ("Long context"). */
  QD_ERR_CONTEXT_CEILING = 3,
  /* A required weight pointer is NULL ("Errors", checkpoint_not_found). */
  QD_ERR_CHECKPOINT_NOT_FOUND = 4,
  /* A caller buffer is smaller than qd_query_sizes() asked for. */
  QD_ERR_BUFFER_TOO_SMALL = 5,
  /* A HIP runtime call failed, or no gfx950 device is present. */
  QD_ERR_DEVICE = 6,
  /* The quantized weight cache is absent or fails its validity gate ("The quantized
   * load cache"): load with qd_load_weights and write a fresh cache. */
  QD_ERR_CACHE_MISS = 7,
} qd_status;

#define QD_MAX_CONTEXT 65536

/* Model dimensions; field names follow the checkpoint's config.json.
 * Gates from "Model-agnostic LLM inference", section "Supported models":
 *   n_heads % n_kv_heads == 0; hidden, intermediate and n_heads*head_dim each a
 *   multiple of 32; tie_word_embeddings != 0; attention_bias == 0.
 * Gates this library adds for its kernels: every size > 0; head_dim a power of
 * two in [32, 256]; vocab >= 2; n_heads / n_kv_heads <= 8. */
typedef struct {
  int32_t hidden;        /* hidden_size */
  int32_t n_layers;      /* num_hidden_layers */
  int32_t n_heads;       /* num_attention_heads */
  int32_t n_kv_heads;    /* num_key_value_heads */
  int32_t head_dim;      /* head_dim */
  int32_t intermediate;  /* intermediate_size */
  int32_t vocab;         /* vocab_size */
  float rms_eps;         /* rms_norm_eps */
  float rope_theta;      /* rope_theta */
  int32_t tie_word_embeddings;
  int32_t attention_bias;
} qd_model_shape;

/* Limits the buffers are sized for. */
typedef struct {
  int32_t max_batch;           /* sequences decoded together, 1..64 */
  int32_t max_ctx;             /* positions per sequence, 1..QD_MAX_CONTEXT */
  int32_t max_prefill_tokens;  /* prompt tokens summed over one qd_prefill call, 1..4000000 */
} qd_limits;

typedef struct {
  uint64_t weight_bytes;     /* int8 codes, fp32 scales and gains, RoPE table */
  uint64_t kv_bytes;         /* bf16 K and V: layers x max_batch x kv_heads x max_ctx x head_dim x 2 */
  uint64_t workspace_bytes;  /* activations, attention partials, counters */
  uint64_t packed_model_bytes; /* int8 + one fp32 scale per row + fp32 gains, embedding once */
} qd_sizes;

/* fp32 weights of one layer in checkpoint layout: row-major [out, in], device
 * pointers.  q [H*D, d], k and v [KV*D, d], o [d, H*D], gate and up [I, d],
 * down [d, I]; gains in_norm and post_norm [d], q_norm and k_norm [D]. */
typedef struct {
  const float *q, *k, *v, *o, *gate, *up, *down;
  const float *in_norm, *post_norm, *q_norm, *k_norm;
} qd_layer_f32;

/* All fp32 weights.  embed [V, d] device pointer (also the LM head: tied),
 * final_norm [d] device pointer, layers: host array of n_layers entries. */
typedef struct {
  const float* embed;
  const float* final_norm;
  const qd_layer_f32* layers;
} qd_weights_f32;

/* Caller-owned device buffers, each at least the size qd_query_sizes() gives,
 * 256-byte aligned. */
typedef struct {
  void* weights;   uint64_t weight_bytes;
  void* kv;        uint64_t kv_bytes;
  void* workspace; uint64_t workspace_bytes;
} qd_buffers;

typedef struct qd_model qd_model;

/* Timing of the last qd_generate_greedy call, from HIP events on its stream. */
typedef struct {
  double prefill_us;   /* prompt processing up to the first generated id */
  double decode_us;    /* the max_new_tokens - 1 decode steps */
  int32_t steps;       /* decode steps run */
  int32_t n_prompt_tokens;
} qd_stats;

/* Message for the last failing call on this thread ("" if none). */
const char* qd_last_error(void);

/* Checks the architecture gates on the host only (no GPU work).  Returns
 * QD_ERR_UNSUPPORTED_ARCH naming every failed gate, or QD_OK. */
qd_status qd_check_shape(const qd_model_shape* shape);

/* Byte sizes of the three caller buffers for a shape and limits (host only).
 * QD_ERR_CONTEXT_CEILING if limits->max_ctx > QD_MAX_CONTEXT. */
qd_status qd_query_sizes(const qd_model_shape* shape, const qd_limits* limits, qd_sizes* out);

/* Validates everything on the host, then quantizes every projection and the
 * embedding on the GPU (per-row absmax / 127, round-half-even, bit-exact with
 * an IEEE fp32 reference) into buffers->weights, builds the RoPE table and
 * clears the KV positions.  The fp32 inputs may be freed once the stream has
 * passed this call.  On success *out is a new handle.
 * Quantization: "Model-agnostic LLM inference", section "The quantized load cache". */
qd_status qd_load_weights(const qd_model_shape* shape, const qd_limits* limits,
                          const qd_weights_f32* weights, const qd_buffers* buffers,
                          qd_stream stream, qd_model** out);

/* Quantized load cache ("Model-agnostic LLM inference", section "The quantized load
 * cache"): the exact post-quantization device bytes, restored instead of re-quantizing.
 * File: a 128-byte little-endian header, then the payload.
 *   header: char magic[8] = "QDI8WCV1"; uint32 version = 2; uint32 header_bytes = 128;
 *           uint64 payload_bytes; uint32 dims[9] = hidden, n_layers, n_heads,
 *           n_kv_heads, head_dim, intermediate, vocab, bit pattern of rms_eps, bit
 *           pattern of rope_theta; uint8 source_digest[32]; uint8 payload_digest[32];
 *           uint8 pad[4].
 *   payload_digest = SHA-256 of the concatenated SHA-256 digests of the payload's
 *           consecutive 16 MiB chunks (the last chunk shorter), so the chunks can be hashed
 *           on several threads.
 *   payload: embedding codes [V, d] int8, embedding scales [V] fp32, final gain [d]
 *           fp32, then per layer: q|k|v codes [H*D + 2*KV*D, d] and scales, O codes
 *           [d, H*D] and scales, gate/up codes [2I, d] and scales (interleaved in blocks
 *           of 16 rows: 16 gate rows, then the matching 16 up rows), down codes [d, I] and
 *           scales, gains input [d], post-attention [d], q_norm [D], k_norm [D].
 * The validity gate: magic, version, every dimension, the caller's 32-byte digest of the
 * source checkpoint (e.g. SHA-256 of its manifest), the exact file length, and the
 * payload digest.  Any mismatch returns QD_ERR_CACHE_MISS naming it, and the
 * caller falls back to qd_load_weights + qd_save_cache. */

/* Writes m's quantized weights to `path` (through `path`.tmp, then a rename).  Host
 * memory: one payload-sized buffer.  Synchronizes `stream`. */
qd_status qd_save_cache(qd_model* m, const char* path, const uint8_t* source_digest,
                        qd_stream stream);

/* As qd_load_weights, but the weights come from a cache file that passes the gate (the
 * RoPE table and device state are rebuilt).  The caller's buffers as for qd_load_weights. */
qd_status qd_load_cache(const qd_model_shape* shape, const qd_limits* limits, const char* path,
                        const uint8_t* source_digest, const qd_buffers* buffers,
                        qd_stream stream, qd_model** out);

/* The gate alone, on the host (no GPU): QD_OK if `path` would load for this shape and
 * digest, else QD_ERR_CACHE_MISS naming what differs. */
qd_status qd_check_cache(const qd_model_shape* shape, const char* path,
                         const uint8_t* source_digest);

/* SHA-256 (FIPS 180-4) of n bytes of host memory into out32[32]. */
qd_status qd_sha256(const void* data, uint64_t n, uint8_t* out32);

/* Identifiers of quantized tensors for qd_export_quantized. */
typedef enum {
  QD_T_EMBED = 0, QD_T_Q = 1, QD_T_K = 2, QD_T_V = 3, QD_T_O = 4,
  QD_T_GATE = 5, QD_T_UP = 6, QD_T_DOWN = 7,
} qd_tensor;

/* Copies one quantized matrix back in checkpoint layout: codes [rows, cols] int8
 * and scales [rows] fp32, to HOST memory.  Synchronizes the stream.  For
 * bit-exact checks of the quantizer. */
qd_status qd_export_quantized(qd_model* m, int32_t tensor, int32_t layer,
                              int8_t* codes_host, float* scales_host, qd_stream stream);

/* Prefill ("LLM inference overview", section "Workload characteristics"): runs
 * n_seqs prompts, concatenated in ids_dev (device, int32, sum(lens) ids), with
 * lengths lens_host[n_seqs] (host), into KV slots 0..n_seqs-1 starting at
 * position 0.  Resets those slots' lengths to their prompt lengths.  Writes the
 * greedy id of each prompt's last row to next_ids_dev[n_seqs] (device) and, if
 * logits_dev is not NULL, that row's fp32 logits to logits_dev[n_seqs, V].
 * Ids are validated on the host (ids_host may be given for that; if NULL the ids
 * are not range-checked). */
qd_status qd_prefill(qd_model* m, int32_t n_seqs, const int32_t* ids_dev,
                     const int32_t* ids_host, const int32_t* lens_host,
                     float* logits_dev, int32_t* next_ids_dev, qd_stream stream);

/* One decode step ("LLM inference overview", section "Workload characteristics": decode
 * produces one token per sequence per step and sweeps every weight once for all B
 * sequences; "Model-agnostic LLM inference", section "Notes": the greedy id is the fused
 * arg-max of the step's logits) for slots 0..B-1: feeds in_ids_dev[B] (device) at each slot's
 * current length p, appends K/V at p, increments p, writes the greedy ids to
 * next_ids_dev[B] and, if logits_dev is not NULL, fp32 logits [B, V].  Teacher
 * forcing is the caller choosing in_ids.  No host synchronization; the slot
 * lengths live on the device.  Returns QD_ERR_INVALID_ARGUMENTS if B is out of
 * range; the caller must not step a slot past max_ctx. */
qd_status qd_decode_step(qd_model* m, int32_t B, const int32_t* in_ids_dev,
                         float* logits_dev, int32_t* next_ids_dev, qd_stream stream);

/* Continuous batching ("LLM inference overview", section "Results": batched decode
 * serves many independent sequences with the weights swept once per step, and sequences
 * join and leave the running batch).  The two calls below address KV slots explicitly,
 * so a new prompt can be prefilled into a free slot while other slots are mid-decode.
 *
 * qd_prefill_slots: as qd_prefill, but prompt b goes to KV slot slots_host[b] (host,
 * n_seqs distinct values in [0, max_batch)); that slot's length is reset to lens_host[b]
 * and its earlier contents are overwritten.  Other slots are untouched.
 * Errors: QD_ERR_INVALID_ARGUMENTS (NULL slots_host, a slot out of range or listed
 * twice, plus every check of qd_prefill), before any GPU work. */
qd_status qd_prefill_slots(qd_model* m, int32_t n_seqs, const int32_t* slots_host,
                           const int32_t* ids_dev, const int32_t* ids_host,
                           const int32_t* lens_host, float* logits_dev, int32_t* next_ids_dev,
                           qd_stream stream);

/* qd_decode_step_slots: one decode step for the B slots slots_host[0..B-1] (host,
 * distinct, each holding a prompt), in any order and at their own lengths: row b of
 * in_ids_dev[B], next_ids_dev[B] and logits_dev[B, V] (nullable) belongs to slot
 * slots_host[b].  Appends K/V at each slot's length p and increments it.  The slot
 * list is staged through pinned host memory on `stream`; no host synchronization.
 * Errors: QD_ERR_INVALID_ARGUMENTS (NULL slots_host, a slot out of range, listed twice,
 * empty or full), before any GPU work. */
qd_status qd_decode_step_slots(qd_model* m, int32_t B, const int32_t* slots_host,
                               const int32_t* in_ids_dev, float* logits_dev,
                               int32_t* next_ids_dev, qd_stream stream);

/* Sampled decode ("Model-agnostic LLM inference", section "Sampling"): the chain
 * repetition / presence / frequency penalties -> temperature -> top-k -> min-p -> top-p
 * -> seeded weighted draw.  Penalties use the occurrences of each token in the sequence
 * so far (its prompt and every token fed since, counted on the device by the prefill and
 * decode calls; a prefill restarts its slots' counts).  A seen token's logit is divided
 * by repeat_penalty when positive and multiplied by it otherwise, then presence_penalty
 * + frequency_penalty * count is subtracted; all logits are divided by temperature.
 * top_k keeps the k largest (equal values: lower id first); min_p keeps probabilities
 * >= min_p x the largest; top_p the shortest prefix of the rest holding top_p of its
 * mass (at least one token).  The draw: u in [0, 1) from Philox4x64-10 with key
 * (seed, 0) and counter (n, 0, 0, 0), n = tokens already drawn for the sequence (reset by
 * its prefill), u = top 24 bits of the first word x 2^-24; the first candidate whose
 * cumulative weight exceeds u x the kept weight is drawn.  Same prompt, parameters and
 * seed give the same tokens; top_k = 1 gives the greedy id (of the penalized logits). */
typedef struct {
  float temperature;        /* > 0 */
  int32_t top_k;            /* 1..1024 (this library's limit) */
  float min_p;              /* [0, 1]; 0 keeps all */
  float top_p;              /* (0, 1]; 1 keeps all */
  float repeat_penalty;     /* > 0; 1 = none */
  float presence_penalty;   /* 0 = none */
  float frequency_penalty;  /* 0 = none */
} qd_sampling;

/* Draws one token per row from logits_dev [B, V] (device, fp32; e.g. the logits output
 * of qd_prefill / qd_decode_step / their _slots forms) for the sequences in KV slots
 * slots_host[b] (host, distinct; NULL: slots 0..B-1), with per-row seeds seeds_host[B]
 * (host).  Writes next_ids_dev[B] (device) and advances each slot's draw number.  The
 * caller feeds the drawn ids to the next decode step.  Asynchronous on `stream`.
 * Errors: QD_ERR_INVALID_ARGUMENTS (a parameter out of range, a NULL pointer, a slot out
 * of range, listed twice or holding no prompt), before any GPU work. */
qd_status qd_sample(qd_model* m, int32_t B, const int32_t* slots_host, const qd_sampling* params,
                    const uint64_t* seeds_host, const float* logits_dev, int32_t* next_ids_dev,
                    qd_stream stream);

/* qd_sample for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid it.  Same
 * arguments, checks, kernels and results as qd_sample; the per-call scratch (penalized
 * rows, histograms, candidate lists, counters, the staged seeds and slot list) lives in a
 * fixed device array of the library (9 MiB + 17 KiB per device, held until the process
 * ends) instead of the model's workspace, so nothing is allocated or freed.  Limits of
 * that array: B <= 16 and B x vocab <= 2,097,152 (at vocab 151,936: 13 rows); larger
 * calls return QD_ERR_INVALID_ARGUMENTS naming the limit, before any GPU work.  Every
 * call on one device shares the array: calls that overlap on one GPU (another stream,
 * another model, another thread) race and must be ordered by the caller. */
qd_status qd_sample_noalloc(qd_model* m, int32_t B, const int32_t* slots_host,
                            const qd_sampling* params, const uint64_t* seeds_host,
                            const float* logits_dev, int32_t* next_ids_dev, qd_stream stream);

/* One call, start to finish ("Model-agnostic LLM inference", section "Notes"):
 * prefill of B prompts (host ids, concatenated; lens_host[B]) then
 * max_new_tokens - 1 decode steps, greedy ids kept on the device between steps:
 * each step is replayed from a captured HIP graph.  out_ids_host[B * max_new_tokens] receives
 * the generated ids (row b = sequence b); n_out_host[b] the count up to and
 * including the first eos_id (eos_id < 0 disables the stop).  Synchronizes the
 * stream once at the end.  stats may be NULL. */
qd_status qd_generate_greedy(qd_model* m, int32_t B, const int32_t* prompt_ids_host,
                             const int32_t* lens_host, int32_t max_new_tokens, int32_t eos_id,
                             int32_t* out_ids_host, int32_t* n_out_host, qd_stats* stats,
                             qd_stream stream);

/* Kernel classes of one decode step, for qd_profile_kernels. */
typedef enum {
  QD_PROF_EMBED = 0, QD_PROF_QKV = 1, QD_PROF_ATTN = 2, QD_PROF_O = 3,
  QD_PROF_GATEUP = 4, QD_PROF_DOWN = 5, QD_PROF_LMHEAD = 6, QD_PROF_COUNT = 7,
} qd_prof_kernel;

/* Measurement aid (not part of the forward pass): launches each decode-step kernel
 * class `iters` times back to back for slots 0..B-1 at their current positions,
 * cycling through the layers (so weights and KV rows come from memory as in a real
 * step), bracketed by HIP events on `stream`, and writes the mean microseconds per
 * launch to us_out[QD_PROF_COUNT] (the LM head and embedding have one instance).  The residual and
 * activation buffers are overwritten (run it after the outputs of interest are
 * read); positions and generated ids are left unchanged.  Synchronizes the stream. */
qd_status qd_profile_kernels(qd_model* m, int32_t B, int32_t iters, float* us_out,
                             qd_stream stream);

/* Launch-policy knobs (performance only; results stay within the parity bar). */
typedef enum {
  QD_TUNE_ATTN_MAX_SPLITS = 0,    /* most position splits per (sequence, KV head); default 64 */
  QD_TUNE_ATTN_MIN_CHUNKS = 1,    /* fewest 64-position chunks per split; default 1 */
  QD_TUNE_ATTN_WAVES = 2,         /* decode-attention waves per work-group: 4, 8, or 0 = by batch (default) */
  QD_TUNE_ATTN_MERGE_LAST = 3,    /* 1 (default): the last split merges in-kernel, except that a
                                     single-row step with 2..8 splits leaves the partials to the
                                     O projection, which merges them as it loads its input;
                                     2: the last split always merges; 0: a merge launch */
  /* 4 and 5 are not used (unknown knobs) */
  QD_TUNE_SKINNY_SPLIT = 6,       /* batched decode projections split K over work-groups:
                                     1 never, 2 (default) projections with fewer than 128
                                     16-channel tiles at batches over 16, 3 all */
  QD_TUNE_GEMM_SPLITS = 7,        /* prefill GEMMs: most split-K ways, 1..8, or 0 (default: 8;
                                     the launcher splits only while the tiles leave CUs idle) */
  QD_TUNE_ATTN_OCCUPANCY = 8,     /* decode attention: splits target this many work-groups per
                                     CU over all (row, KV head) pairs, 1..8, or 0 (default: as
                                     many as stay resident, 1 for 8 waves, 3 for 4 waves) */
  QD_TUNE_SKINNY_NORM = 9,        /* batched decode: 1 (default) folds the RMSNorm before q|k|v
                                     and gate|up into the projection where the shape allows;
                                     0: a separate normalization launch */
  QD_TUNE_PREFILL_GEMM = 10,      /* prefill GEMMs: 1 (default) the k-sliced kernel for few
                                     token rows and, for more rows, QK-norm / RoPE / K/V cache
                                     writes in the q|k|v GEMM's epilogue where the shapes allow;
                                     0: the k-stepped kernel and a separate QK-norm launch */
  QD_TUNE_SKINNY_XSTAGE = 11,     /* batched decode projections of 2..16 rows, and those with
                                     the RMSNorm folded in at 9..32 rows: 1 (default) load
                                     activation rows contiguously and reorder them through LDS;
                                     0: load them directly in the matrix-core operand layout */
  QD_TUNE_FLASH_ROWS = 12,        /* prefill attention query rows per work-group: 64, 128 (head
                                     dim up to 128), or 0 (default: 128 when those tiles give
                                     every CU two work-groups) */
} qd_tune_knob;

/* Sets a knob; captured decode graphs are dropped so the next call re-captures.
 * QD_ERR_INVALID_ARGUMENTS for an unknown knob or a value out of its range. */
qd_status qd_set_tuning(qd_model* m, int32_t knob, int32_t value);

/* Kernel classes of a decode step, for qd_run_op. */
typedef enum {
  QD_OP_EMBED = 0, QD_OP_QKV = 1, QD_OP_O = 2, QD_OP_GATEUP = 3, QD_OP_DOWN = 4,
  QD_OP_LMHEAD = 5, QD_OP_COUNT = 6,
} qd_op;

/* Test aid (not part of the forward pass): runs one kernel class of a decode step for B
 * rows, launched exactly as qd_decode_step launches it at that B (the same kernels, tile
 * shapes and work splits), on caller-given device inputs of `layer`'s weights:
 *   QD_OP_EMBED   in: token ids int32 [B]              out: bf16 [B, hidden] = code x row scale
 *   QD_OP_QKV     in: residual bf16 [B, hidden]        out: bf16 [B, H*D + 2*KV*D] (q | k | v)
 *                 of RMSNorm(in, input gain), projected (the norm runs inside the projection)
 *   QD_OP_O       in: attention output bf16 [B, H*D], resid: bf16 [B, hidden]
 *                 out: bf16 [B, hidden] = resid + projection
 *   QD_OP_GATEUP  in: residual bf16 [B, hidden]        out: bf16 [B, intermediate] =
 *                 SiLU(gate) x up of RMSNorm(in, post-attention gain)
 *   QD_OP_DOWN    in: bf16 [B, intermediate], resid: bf16 [B, hidden]
 *                 out: bf16 [B, hidden] = resid + projection
 *   QD_OP_LMHEAD  in: residual bf16 [B, hidden]        out: fp32 logits [B, vocab] of
 *                 RMSNorm(in, final gain) against the tied embedding; ids_out: int32 [B], the
 *                 fused arg-max (lowest index among equal maxima)
 * All pointers are device pointers, rows dense; resid is read for QD_OP_O and QD_OP_DOWN only,
 * ids_out for QD_OP_LMHEAD only (required there).  Overwrites the workspace's activation
 * buffers; KV cache, positions and sampler state are left unchanged.  Asynchronous on
 * `stream`.  QD_ERR_INVALID_ARGUMENTS for an unknown op, a layer or B out of range or a NULL
 * pointer, before any GPU work.  Its purpose is exact checks of each projection kernel:
 * with integer-valued codes whose row maximum is 127 (scale exactly 1) and integer-valued
 * inputs, every fp32 accumulator is an exact integer in any summation order. */
qd_status qd_run_op(qd_model* m, int32_t op, int32_t layer, int32_t B, const void* in_dev,
                    const void* resid_dev, void* out_dev, int32_t* ids_out_dev, qd_stream stream);

/* Frees the handle's host state and captured graphs ("Model-agnostic LLM inference",
 * section "Notes": weights stay resident across calls until the model is released).
 * The caller's device buffers remain the caller's; NULL is a no-op. */
void qd_free(qd_model* m);

#ifdef __cplusplus
}
#endif
#endif /* QD_H */
