/*
 * qdec.h -- C ABI of the MI355X decoder library (libqdec.so).
 *
 * The library runs the forward pass of a Llama / Qwen3 / Gemma-3-style decoder
 * over GGUF block-quantized weights on one gfx950 GPU: prefill of a prompt and
 * token-by-token decode over a KV cache, with greedy or temperature sampling.
 *
 * What each call computes is defined on these pages:
 *   [W]  "How Modern LLMs Actually Generate Text: A Pure Python Walkthrough"
 *        (Qwen3-0.6B in MLX), Steps 2-9: embedding, RMSNorm, RoPE, grouped-query
 *        attention with a KV cache, SwiGLU, the block, LM head, sampling, the
 *        generation loop.
 *   [S]  Synsema "Local inference and architectures": the qwen3 architecture
 *        file (op order, per-head Q/K norm before RoPE, tied head
 *        `output.weight | token_embd.weight`), gelu_tanh for Gemma 3, and the
 *        rule that weights stay block-quantized and are multiplied in f32.
 *   [T]  tessl `python/README.md`, sections "Handle ownership, closing and
 *        errors" and "How the buffers cross": opaque handle freed exactly once,
 *        status 1 = refusal / status 2 = bug caught at the boundary, a poisoned
 *        latch after GPU failure, waiting for in-flight work on failure.
 *   [P]  "PyTensor Beyond PyMC: Building LLM Inference in Python": its
 *        engineering-roadmap table (a paged KV cache and continuous batching)
 *        and its Q4_K_M GGUF file.
 *
 * Conventions for every call:
 *   - `d_*` arguments are device pointers on the current HIP device; other
 *     pointers are host pointers.  The library never frees caller memory.
 *   - `stream` is a hipStream_t (may be NULL for the null stream).  Work is
 *     enqueued on it and the call returns without a host wait, except where a
 *     call says otherwise.  Caller buffers must stay alive until the stream has
 *     passed the call.
 *   - Return value: QDEC_OK, QDEC_REFUSED (caller error found before anything
 *     was enqueued; the handle stays usable; qdec_last_error() says which
 *     argument and why), or QDEC_INTERNAL (a HIP error or a broken internal
 *     invariant; the library drained the stream with a bounded wait and
 *     latched the handle as poisoned: every later call on it is refused until
 *     it is freed).
 *   - A handle is used from one thread at a time; error text is thread-local.
 */
#ifndef QDEC_H
#define QDEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDEC_ABI_VERSION 5

enum { QDEC_OK = 0, QDEC_REFUSED = 1, QDEC_INTERNAL = 2 };

/* Tensor types, numbered as a GGUF file numbers them (ggml type ids).
 * Q8_0: 34-byte blocks = fp16 scale d + 32 int8 q, w = d*q.
 * Q4_0: 18-byte blocks = fp16 scale d + 16 bytes; byte j holds element j in its
 *       low nibble and element j+16 in its high nibble, w = d*(n-8).
 * Blocks run along a row's input dimension; a row holds ceil(cols/32) blocks.
 * Q4_K, Q6_K (the K-quants of GGUF files such as Q4_K_M): 256-value
 *       super-blocks of 144 / 210 bytes in GGUF's layout; rows hold cols/256 of
 *       them (cols a multiple of 256).  Q4_K: fp16 d, fp16 dmin, eight 6-bit
 *       (scale, min) pairs, w = d*sc*q - dmin*m; Q6_K: 6-bit q, sixteen int8
 *       scales, fp16 d, w = d*scale*(q - 32).  They are repacked at load into
 *       32-value blocks that keep the file's scales unpacked to whole bytes
 *       (0.578 and 1.078 bytes per weight against the file's 0.5625 and
 *       0.8203) and stream as such. */
enum { QDEC_T_F32 = 0, QDEC_T_Q4_0 = 2, QDEC_T_Q8_0 = 8, QDEC_T_Q4_K = 12, QDEC_T_Q6_K = 14 };

enum { QDEC_ACT_SILU = 0, QDEC_ACT_GELU_TANH = 1 };

/* Operand precision of the prefill projections (quantized weights; f32 weights
 * always use f32 operands).  F32: f32 operands on V_MFMA_F32_32X32X2_F32, the
 * [S] "Choose the engine" contract (weights decoded exactly, products in f32).
 * BF16X3: quant values (exact in bf16) against a three-term bf16 split of the
 * activations, x = x1 + x2 + x3 with 8 significant bits each, on
 * V_MFMA_F32_32X32X16_BF16: every product is exact and accumulated in f32, so
 * the result is the f32 one up to summation order.  BF16: activations rounded
 * to bf16 (one term); not f32-accurate.  Projections with too few 64 x 128
 * tiles to fill the GPU keep the f32 K-split kernel in every mode. */
enum { QDEC_PREFILL_F32 = 0, QDEC_PREFILL_BF16X3 = 1, QDEC_PREFILL_BF16 = 2 };

enum {
  QDEC_ALL_LOGITS = 1u << 0,       /* prefill: logits of every position, not only the last */
  QDEC_TOKENS_ON_DEVICE = 1u << 1  /* decode: `tokens` is a device pointer (e.g. last d_token_out) */
};

typedef struct qdec_model qdec_model; /* opaque; owned by the caller; freed exactly once */

/* Model shape.  [W] Steps 3-7 and [S] "The format" define the block; window /
 * window_period / rope_theta_local / sandwich_norm / act cover the Gemma-3
 * variant: layer i uses full attention and rope_theta iff
 * window == 0 or i % window_period == window_period - 1, otherwise keys with
 * p - window < j <= p and rope_theta_local. */
typedef struct {
  int32_t n_layer, hidden, n_head, n_head_kv, head_dim, ffn, vocab;
  float rms_eps, rope_theta, rope_theta_local;
  int32_t window, window_period;
  int32_t qk_norm;       /* per-head RMSNorm of q and k (gain [head_dim]) before RoPE */
  int32_t sandwich_norm; /* RMSNorm of each sublayer output before its residual add */
  int32_t act;           /* QDEC_ACT_* */
  int32_t qkv_bias;      /* q, k and v projections add a bias vector ([S] "The format": the
                            qwen2 architecture differs from llama by these three bias adds);
                            tensors blk.i.attn_{q,k,v}.bias, F32, rows = 1 */
} qdec_config;

/* One tensor in GGUF naming ("token_embd.weight", "blk.3.attn_q.weight",
 * "blk.3.attn_q_norm.weight", "blk.3.post_attention_norm.weight",
 * "blk.3.post_ffw_norm.weight", "blk.3.attn_q.bias", "output_norm.weight",
 * "output.weight", ...).
 * Matrices are [rows = output dim][cols = input dim]; 1-D gains and biases have
 * rows = 1, type QDEC_T_F32.  host_data is borrowed for the duration of the call. */
typedef struct {
  const char* name;
  int32_t type;
  int64_t rows, cols;
  const void* host_data;
  int64_t n_bytes; /* rows*ceil(cols/32)*{34|18}, rows*(cols/256)*{144|210}, or rows*cols*4 (F32) */
} qdec_tensor;

int32_t qdec_abi_version(void);
const char* qdec_last_error(void); /* valid until the next call on this thread */

/* Validate every tensor (names required by cfg, types, dims, byte counts,
 * finite fp16 scales) before allocating anything; then copy the weights into
 * library-owned device memory, repacked to an aligned scale/quant split with the
 * same byte count, and allocate an f32 KV cache of max_seqs x max_ctx
 * positions.  `output.weight` is optional (absent: the head reuses
 * token_embd.weight, [S] `a | b`).  Synchronizes `stream` before returning.
 * Limits: 1 <= max_seqs <= 64; hidden and head_dim multiples of 32 and head_dim
 * in {64, 128, 256}; n_head a multiple of n_head_kv; fewer than 2^31 cache rows
 * per layer (max_seqs * n_head_kv * max_ctx). */
int qdec_load_weights(const qdec_config* cfg, const qdec_tensor* tensors, int32_t n_tensors,
                      int32_t max_seqs, int32_t max_ctx, void* stream, qdec_model** out);

/* Model files.  `path` names a GGUF file (the public GGUF container, versions 2
 * and 3, little-endian; tensors named as in qdec_tensor); `archdef` is the text
 * of an architecture definition in the format of [S] "The format" (header
 * `arch` / `kind decoder` / `param`, sections prologue, block (per layer, {i}),
 * epilogue; `dst = op(...)` or `op(dst, ...)`; `a | b`), or NULL for the
 * built-in definition of the file's general.architecture (llama, qwen2, qwen3,
 * gemma3: qdec_archdef_builtin).  The definition is compiled, not interpreted:
 * each statement is evaluated symbolically and what the block computes must be
 * one of the layouts the kernels run -- llama's pre-norm block with a silu or
 * gelu_tanh gate, optionally with q/k/v biases, per-head q/k norms before RoPE,
 * and sandwich norms; the prologue must be x = embed(token_embd.weight) and the
 * epilogue logits = matmul(last(rms_norm(x, output_norm.weight)), output.weight
 * | token_embd.weight).  Anything else is refused with the reason.  Every name
 * a statement uses must resolve, in statements whose results are never used
 * too: a tensor (one of its `|` alternatives; for the block, in every layer)
 * must be in the file, a number argument must be head_count, head_count_kv, a
 * finite number or an <arch>. metadata key of the file, and {i} may appear only
 * in the block.
 * Shape from the metadata of the definition's arch: <arch>.block_count,
 * .embedding_length, .feed_forward_length, .attention.head_count,
 * .attention.head_count_kv (default head_count), .attention.key_length
 * (default embedding_length / head_count; value_length must equal it),
 * .attention.layer_norm_rms_epsilon, .rope.freq_base (default 10000),
 * .attention.sliding_window (default 0); vocab = rows of token_embd.weight.  A
 * file with a window needs the definition's `param window_pattern P` (layer i
 * is global iff i % P == P - 1); `param rope_freq_base_local B` sets the
 * rotary base of window layers (default: the global one).  general.architecture
 * must equal the definition's arch.
 * qdec_gguf_config: the config only; no GPU work.  Status 1 on any refusal. */
int qdec_gguf_config(const char* path, const char* archdef, qdec_config* out);

/* qdec_gguf_config, then qdec_load_weights over the tensors the compiled
 * layout reads, borrowed from a read-only mapping of the file until the weights
 * are on the device.  Tensor types F32, Q4_0, Q8_0, Q4_K, Q6_K; a quantized row
 * holds whole blocks (32 values; 256 for the K-quants).  Other tensors in the
 * file are ignored. */
int qdec_load_gguf(const char* path, const char* archdef, int32_t max_seqs, int32_t max_ctx, void* stream,
                   qdec_model** out);

/* Text of the built-in definition of `arch` (static storage), or NULL. */
const char* qdec_archdef_builtin(const char* arch);

/* Prefill ([W] Step 9, phase 1): append n_tokens host token ids at positions
 * kv_len(seq).. and advance kv_len(seq) by n_tokens.  Writes logits f32 [vocab]
 * of the last position (or [n_tokens][vocab] with QDEC_ALL_LOGITS) to d_logits,
 * and the greedy token of the last position to d_token_out if non-NULL.
 * Refused: seq out of range, n_tokens <= 0, kv_len + n_tokens > max_ctx, a token
 * outside [0, vocab), NULL d_logits. */
int qdec_prefill(qdec_model* m, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                 float* d_logits, int32_t* d_token_out, uint32_t flags, void* stream);

/* Decode step ([W] Step 9, phase 2): sequences 0..n_seqs-1 each consume
 * tokens[s] at position kv_len(s), which then advances by one.  Writes logits
 * f32 [n_seqs][vocab] and the chosen tokens int32 [n_seqs].  temperature == 0:
 * greedy argmax (lowest index on ties); temperature > 0: argmax of
 * logits/temperature + Gumbel noise from Philox4x64-10 with key (seed, 0) and
 * counter (v/4, step, s, 0), word v%4, u = ((r>>41)+0.5)*2^-23.
 * top_p < 1 with temperature > 0 restricts the draw to the nucleus ([W] Step 8
 * sampler): with p = softmax(logits/temperature) sorted descending (equal
 * logits by lower index), the first count(running sum < top_p) + 1 tokens
 * (top_p <= 0: the first token).  The running sums use per-token weights
 * floor(2^40 * 2^((l - max l) * log2(e) / temperature)) (f32) summed exactly;
 * a row with a non-finite logit keeps every token.  top_p >= 1: no restriction.
 * Decode attention combines its position chunks with f32 atomic adds, and 5..16
 * rows run some projections with K split across workgroups the same way, so
 * repeated steps agree with each other to f32 rounding, not bit for bit.
 * With QDEC_TOKENS_ON_DEVICE, tokens is a device pointer; ids outside [0, vocab)
 * are clamped and latch a host-mapped error word: the first call made after
 * the stream has run that step returns QDEC_INTERNAL and poisons the handle.
 * Refused: n_seqs outside [1, max_seqs], any kv_len(s) == max_ctx, a host token
 * out of range, temperature < 0 or NaN, top_p NaN, NULL outputs. */
int qdec_decode_step(qdec_model* m, const int32_t* tokens, int32_t n_seqs, float* d_logits,
                     int32_t* d_token_out, float temperature, float top_p, uint64_t seed,
                     uint64_t step, uint32_t flags, void* stream);

/* Continuous batching ([P] "PyTensor Beyond PyMC: Building LLM Inference in
 * Python", engineering-roadmap table, KV-cache row: continuous batching; [W]
 * Step 9's loop, run for several sequences): one decode step for an arbitrary
 * set of sequence slots, so sequences can join and leave between steps.  Row r
 * of tokens / d_logits / d_token_out serves sequence seqs[r] (host array of n
 * distinct slots in [0, max_seqs)) at position kv_len(seqs[r]).  The random
 * stream of row r is sequence seqs[r]'s (Philox counter (v/4, step, seqs[r],
 * 0)), so a sequence's draws do not depend on which others share the step.
 * Otherwise as qdec_decode_step, which is this call with seqs = 0..n-1.
 * Refused: a slot out of range or given twice, and the qdec_decode_step cases. */
int qdec_decode_batch(qdec_model* m, const int32_t* seqs, const int32_t* tokens, int32_t n, float* d_logits,
                      int32_t* d_token_out, float temperature, float top_p, uint64_t seed, uint64_t step,
                      uint32_t flags, void* stream);

/* Paged KV cache ([P], same table row: a paged cache).  Replaces the
 * contiguous max_seqs x max_ctx cache by a pool of n_pages pages of page_size
 * positions shared by all sequences.  Pages are handed out as a sequence grows
 * (qdec_prefill, decode, qdec_kv_write) and returned by qdec_kv_reset /
 * qdec_kv_truncate; a call that needs more pages than are free is refused
 * (status 1) before anything is enqueued.  page_size: a power of two in
 * [16, 2^20], at least the decode chunk (64 positions at head_dim 128, 32 at
 * 256, 128 at 64), and large enough that max_ctx / page_size <= 64.  Every
 * sequence must be empty (status 1 otherwise).  max_ctx still bounds each
 * sequence.  Results are those of the contiguous cache.  Synchronizes stream. */
int qdec_kv_paged(qdec_model* m, int32_t page_size, int32_t n_pages, void* stream);

/* The cache's page size (0 = contiguous), pool size and free pages. */
int qdec_kv_pages(const qdec_model* m, int32_t* page_size, int32_t* n_pages, int32_t* n_free);

/* Ring-buffer cache for sliding-window layers ([P], the same roadmap row: a
 * paged or ring-buffer cache).  A window layer attends to its last `window`
 * positions only, so in the contiguous cache it keeps a ring of R positions,
 * position j in slot j mod R: R is the power of two >= window + P - 1 (P: the
 * positions of one prefill pass, min(max_ctx, 4096), or max_seqs if larger), at
 * least 64, and the ring is used when R <= max_ctx / 2 (enable = 1, the state
 * after load); enable = 0 gives every layer max_ctx positions.  Results are
 * the same either way.  With a ring, qdec_kv_write keeps the last R of the
 * preset positions and qdec_kv_truncate may drop at most R - window positions.
 * Refused (status 1): enable not 0 or 1, a paged cache (pages hold every
 * position), a sequence holding positions.  Synchronizes stream. */
int qdec_kv_ring(qdec_model* m, int32_t enable, void* stream);

/* Positions of layer's ring (0: the layer keeps max_ctx positions, or the cache
 * is paged), written to *out.  Host-side only. */
int qdec_kv_ring_positions(const qdec_model* m, int32_t layer, int32_t* out);

/* Forget the cached positions of one sequence (seq = -1: all), so that its next
 * prefill starts at position 0 ([W] Step 9: each generation starts from an empty
 * cache; a new prompt is a new sequence).  Host-side only, nothing is enqueued;
 * stale KV rows are never read past kv_len.  Refused: seq outside [-1, max_seqs),
 * a poisoned handle. */
int qdec_kv_reset(qdec_model* m, int32_t seq);

/* Roll sequence seq back to its first n positions (0 <= n <= kv_len(seq)), for
 * instance to rerun decode steps over a preset cache.  With window-layer rings
 * (qdec_kv_ring) at most R - window positions may go (status 1 otherwise).
 * Host-side only. */
int qdec_kv_truncate(qdec_model* m, int32_t seq, int32_t n);

/* Install preset post-RoPE K and V, each f32 [n_head_kv][n_pos][head_dim]
 * (device), for one (sequence, layer) at positions 0..n_pos-1, and set
 * kv_len(seq) = n_pos (a window layer's ring keeps the last R of them). */
int qdec_kv_write(qdec_model* m, int32_t seq, int32_t layer, const float* d_k, const float* d_v,
                  int32_t n_pos, void* stream);

/* Number of cached positions of sequence seq ([W] Step 9: the position of the
 * next token), written to *out.  Host-side only.  Refused: NULL pointers, seq out
 * of range. */
int qdec_kv_len(const qdec_model* m, int32_t seq, int32_t* out);

/* Positions per decode-attention chunk and chunks per (sequence, KV head) of the
 * split over positions ([W] Step 5's attention, summed chunk by chunk with an
 * online softmax), as sized at load (and by qdec_kv_paged).  Host-side only. */
int qdec_decode_chunks(const qdec_model* m, int32_t* chunk, int32_t* n_chunks);

/* Operand precision of later prefill projections (QDEC_PREFILL_*; default F32).
 * Refused: an unknown value. */
int qdec_set_prefill_precision(qdec_model* m, int32_t precision);
int qdec_poisoned(const qdec_model* m); /* 1 if latched, 0 if not, -1 for NULL */

/* Release everything the handle owns -- weights, KV cache, workspace, captured
 * graphs -- after draining its last stream (bounded wait, 30 s), as [T]
 * "Handle ownership, closing and errors" requires of a handle's close: work in
 * flight may still read or write the memory.  Call exactly once per handle: a
 * second call is undefined behaviour (there is no registry of live handles).
 * A poisoned handle is freed the same way.  Refused: NULL. */
int qdec_free(qdec_model* m);

/* ---------------------------------------------------------------- tests and measurement */

/* Decode the named tensor (as loaded) to f32 [rows][cols] in d_out: element
 * (r, k) is d * q (Q8_0), d * (n - 8) (Q4_0) or the K-quant forms, one exact
 * f32 product each (an fp16 scale times a small integer needs at most 19
 * significant bits), so any exact decode matches it bit for bit.  This is a
 * separate decode kernel: the projection kernels never form d * q (the GEMV
 * scales each block's dot product, the GEMMs decode their own LDS tiles);
 * qdec_debug_matmul with one-hot input rows checks those bit for bit. */
int qdec_debug_dequant(qdec_model* m, const char* name, float* d_out, void* stream);

/* Embedding gather of n device token ids into d_out f32 [n][hidden]. */
int qdec_debug_embed(qdec_model* m, const int32_t* d_tokens, int32_t n, float* d_out, void* stream);

/* Row-wise token choice over d_logits [rows][vocab] with the decode step's rule
 * (temperature 0: argmax with the lowest index on ties, NaN ranking above every
 * number; else Gumbel-max with counter (v/4, step, row, 0), restricted to the
 * top-p nucleus when top_p < 1).  d_out int32 [rows]. */
int qdec_debug_sample(const float* d_logits, int32_t rows, int32_t vocab, float temperature,
                      float top_p, uint64_t seed, uint64_t step, int32_t* d_out, void* stream);

/* qdec_debug_sample without allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same rule and same kernels as qdec_debug_sample; the
 * partial results live in a fixed file-scope device array of the library
 * (563,712 bytes per GPU, held until the process ends), so rows <= 64 and
 * vocab <= 2^20 (refused otherwise, status 1).  Enqueued on `stream` without a
 * host wait (qdec_debug_sample synchronizes).  Calls that overlap on one GPU --
 * on different streams, or from several threads -- share that array and race:
 * the caller orders them (one stream, or events).  Status 2 on a launch error
 * (no handle is involved, so nothing is poisoned). */
int qdec_sample_noalloc(const float* d_logits, int32_t rows, int32_t vocab, float temperature, float top_p,
                        uint64_t seed, uint64_t step, int32_t* d_out, void* stream);

/* One projection y[r][n] = sum_k W[n][k] x[r][k] with the forward pass's kernels:
 * the decode GEMV for n_x <= 16, the prefill MFMA GEMM above (operands in
 * `precision`, QDEC_PREFILL_*).  W is given in GGUF bytes on the host (uploaded
 * and repacked per call; synchronous).  d_x f32 [n_x][ceil(cols/32)*32] (zero
 * padded), d_y f32 [n_x][rows]. */
int qdec_debug_matmul(int32_t type, int64_t rows, int64_t cols, const void* host_data,
                      int64_t n_bytes, const float* d_x, int32_t n_x, float* d_y, int32_t precision,
                      void* stream);

/* Test hook for the failure path of [T] "Handle ownership, closing and errors"
 * (status 2, drain, poisoned latch).  where = 1 arms it: the next call that
 * launches a kernel enqueues that kernel, then fails as a HIP error would --
 * status QDEC_INTERNAL, the stream drained with the bounded wait, the handle
 * latched as poisoned.  Host-side: no device fault occurs.  where = 0 disarms.
 * Refused: other values, a NULL or poisoned handle. */
int qdec_debug_inject_fault(qdec_model* m, int32_t where);

/* Per-kernel timing with HIP events on the launch stream.  enable = 1 starts
 * recording every launch; enable = 0 synchronizes, writes up to max_out records
 * (one per kernel class) and stops.  Records carry the algorithmic bytes and
 * flops of each launch as the library counts them. */
typedef struct {
  char name[32];
  int64_t launches;
  double total_ms;
  double bytes; /* algorithmic HBM bytes summed over launches */
  double flops; /* algorithmic flops summed over launches */
} qdec_kstat;

int qdec_kernel_timing(qdec_model* m, int32_t enable, qdec_kstat* out, int32_t max_out, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* QDEC_H */
