/*
 * llama_mi355x.h -- C ABI of the MI355X (gfx950) Llama-3 decoder forward pass.
 *
 * The library computes the decoder stack described in the article "250 lines of code to
 * build Llama 3 from scratch" (ai02.cc, a walk-through of naklecha/llama3-from-scratch):
 * token embedding (section 分词器与编码), per layer RMSNorm, Q/K/V projections with
 * rotary position embedding (sections 查询向量, 位置编码, 键向量, 值向量), causal
 * grouped-query attention (sections 查询和键相乘, 掩码, 注意力向量, 多头注意力), the
 * output projection and residual add (section 相加与归一化), the SwiGLU feed-forward
 * and residual add (section 前馈神经网络层), then the final RMSNorm, the vocabulary
 * projection and the greedy argmax (section 预测下一个输出).  Prefill runs a whole prompt;
 * decode runs one token per sequence against a key/value cache pre-allocated by
 * max_seq x max_batch (the cache sizing described on the Hacker News thread "Llama 3
 * implemented in pure NumPy").
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library only
 *    borrows them.  Weights, KV cache and workspace passed to llama_init_weights must stay
 *    valid until llama_free.  The library allocates no device memory.
 *  - Matrices are row-major.  Weights are stored [out_features, in_features] and applied
 *    as x @ W^T, as in the checkpoint (article, section 查询向量).  Q rows are ordered
 *    head * head_dim + i; K and V rows kv_head * head_dim + i.
 *  - Weight element type is the config's dtype: LLAMA_BF16 (bfloat16 weights, KV cache and
 *    GEMM operands, fp32 accumulation, fp32 residual stream and logits) or LLAMA_F32
 *    (every tensor fp32; the debug/reference precision).  Residual-stream tensors
 *    (x_in/x_out) and logits are always fp32; token ids are int32.
 *  - Calls are asynchronous on the given HIP stream (NULL = the null stream).  The library
 *    never synchronises the device except in llama_sync_status.  One model handle must not
 *    be used by two host threads at once, nor by overlapping calls on different streams.
 *  - Every argument, shape and capacity check runs before any device work; on a non-OK
 *    status nothing has been launched, except for LLAMA_ERR_HIP, which reports a failed
 *    launch.  A thread-local message describing the last failure is kept
 *    (llama_last_error).  Cache positions below the call's start position are never
 *    written.
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLAMA_OK = 0,
    LLAMA_ERR_INVALID_ARG = -1, /* null pointer, out-of-range layer, bad token id (device) */
    LLAMA_ERR_SHAPE = -2,       /* inconsistent config or call shape                      */
    LLAMA_ERR_CAPACITY = -3,    /* batch, sequence, token count or buffer size too large   */
    LLAMA_ERR_DTYPE = -4,       /* unknown dtype                                           */
    LLAMA_ERR_HIP = -5,         /* a HIP launch or runtime call failed                     */
    LLAMA_ERR_ALLOC = -6        /* host allocation of the handle failed                    */
} llama_status;

typedef enum { LLAMA_BF16 = 0, LLAMA_F32 = 1 } llama_dtype;

/* Model hyper-parameters (article, section 下载并读取模型权重: dim 4096, n_layers 32,
 * n_heads 32, n_kv_heads 8, vocab 128256, norm_eps 1e-5, rope_theta 500000) and the
 * capacity the caller provisions. */
typedef struct {
    int32_t dim;         /* model width D = n_heads * head_dim                              */
    int32_t n_layers;    /* L                                                               */
    int32_t n_heads;     /* query heads H                                                   */
    int32_t n_kv_heads;  /* key/value heads G; H % G == 0; query head h uses KV head h/(H/G) */
    int32_t head_dim;    /* d, a multiple of 4, <= 256                                        */
    int32_t ffn_hidden;  /* SwiGLU hidden width F (14336 for the 8B shape)                   */
    int32_t vocab_size;  /* V                                                                */
    float norm_eps;      /* RMSNorm epsilon                                                  */
    float rope_theta;    /* RoPE base: theta_i = rope_theta^(-2i/d)                          */
    int32_t max_batch;   /* sequences held in the KV cache                                   */
    int32_t max_seq;     /* positions held per sequence (pos + S <= max_seq)                  */
    int32_t max_tokens;  /* largest B*S of one prefill or layer call                          */
    llama_dtype dtype;   /* weight / cache / operand element type                            */
} llama_config;

/* Device pointers to one layer's weights, names as in the checkpoint
 * (layers.N.attention_norm.weight, layers.N.attention.wq.weight, ...). */
typedef struct {
    const void *attention_norm; /* [D]                          */
    const void *wq;             /* [H*d, D]                     */
    const void *wk;             /* [G*d, D]                     */
    const void *wv;             /* [G*d, D]                     */
    const void *wo;             /* [D, H*d]                     */
    const void *ffn_norm;       /* [D]                          */
    const void *w1;             /* [F, D]  gate                  */
    const void *w3;             /* [F, D]  up                    */
    const void *w2;             /* [D, F]  down                  */
} llama_layer_weights;

typedef struct {
    const void *tok_embeddings;        /* [V, D]                                       */
    const llama_layer_weights *layers; /* HOST array of n_layers entries (copied)      */
    const void *norm;                  /* [D] final RMSNorm weight                      */
    const void *output;                /* [V, D] vocabulary projection (not tied)      */
} llama_weights;

typedef struct llama_model llama_model; /* opaque handle */

/* Bytes of KV cache the caller must provide for this config (layout is internal): keys
 * and values of every layer for max_batch sequences of max_seq positions, the cache the
 * Hacker News thread describes as pre-allocated by max_seq_len x max_batch_size.  0 if
 * the config is invalid (llama_last_error says why). */
size_t llama_kv_cache_bytes(const llama_config *cfg);

/* Bytes of device workspace the caller must provide for this config: the activations of
 * up to max(max_tokens, max_batch) rows between the steps of the article's layer (sections
 * 构建Transformer层 to 前馈神经网络层), the rotary table of section 位置编码, attention
 * partials, split-K sums of the residual GEMMs (the few-row ones, and the down projection of
 * a prefill of up to 4096 rows), device flags.  The largest call is fixed by
 * the config's max_tokens, so the size depends on the config alone.  0 if the config is
 * invalid. */
size_t llama_workspace_bytes(const llama_config *cfg);

/* Validate cfg, borrow the weights, KV cache and workspace, and return a handle in *out.
 * Makes no device call; the RoPE table (cos and sin of m*theta_i for every position m <
 * max_seq, angles formed in double precision, article section 位置编码) is built on the
 * device by the first call that needs it, which also zero-fills the KV cache (attention
 * reads whole 64-position blocks and weights positions past the context by exactly 0, so
 * every cached value must be finite).  kv_bytes and ws_bytes must be at least the
 * sizes above, and both buffers 256-byte aligned.  Errors: INVALID_ARG (null pointers),
 * SHAPE (dim != n_heads*head_dim, H % G != 0, odd or >256 head_dim, non-positive sizes,
 * bf16 dims that are not multiples of 64), DTYPE, CAPACITY (buffers too small), ALLOC. */
llama_status llama_init_weights(const llama_config *cfg, const llama_weights *weights,
                                void *kv_cache, size_t kv_bytes,
                                void *workspace, size_t ws_bytes, llama_model **out);

/* Causal prefill of B independent sequences of S tokens each, starting at position 0
 * (article, sections 分词器与编码 through 预测下一个输出): embeds tokens [B,S], runs every
 * layer (writing the KV cache at positions 0..S-1 of sequences 0..B-1), applies the final
 * RMSNorm and the vocabulary projection.  Writes fp32 logits [B,V] of each sequence's last
 * position, or [B,S,V] of every position when all_positions != 0.  Needs B <= max_batch,
 * S <= max_seq, B*S <= max_tokens.  Equals llama_prefill_at with start_pos 0 and no
 * next_tokens. */
llama_status llama_prefill(llama_model *m, const int32_t *tokens, int32_t B, int32_t S,
                           float *logits, int32_t all_positions, hipStream_t stream);

/* Prefill continued from position start_pos (chunked prefill into an existing cache): the
 * S tokens [B,S] of each of B sequences sit at positions start_pos..start_pos+S-1, their keys
 * and values are written to the cache there, and each attends causally to cache positions
 * 0..its own position, which needs the cache filled at 0..start_pos-1 by earlier calls
 * (article, section 多头注意力 for the causal mask; the cache itself is the Hacker News
 * thread's pre-allocated max_seq_len x max_batch_size buffer).  Logits as llama_prefill.
 * If next_tokens is not NULL it receives int32 [B]: the greedy choice from each sequence's
 * last position, the argmax of its logits with the lowest index on ties (article, section
 * 预测下一个输出).  Needs start_pos >= 0, start_pos + S <= max_seq, B <= max_batch,
 * B*S <= max_tokens; CAPACITY otherwise. */
llama_status llama_prefill_at(llama_model *m, const int32_t *tokens, int32_t B, int32_t S,
                              int32_t start_pos, float *logits, int32_t all_positions,
                              int32_t *next_tokens, hipStream_t stream);

/* One KV-cache decode step: token tokens[b] of sequence b sits at position pos, its key
 * and value are written to the cache at pos, and it attends to cache positions 0..pos
 * (the article's layer, sections 构建Transformer层 to 前馈神经网络层, for one new token;
 * the cache is the Hacker News thread's pre-allocated one).  Writes next_tokens[b] =
 * argmax of its logits (lowest index on ties; article, section 预测下一个输出) and, if
 * logits is not NULL, the fp32 logits [B,V].  Needs B <= max_batch, 0 <= pos < max_seq,
 * and the cache filled at 0..pos-1 by earlier calls.  tokens and next_tokens may alias. */
llama_status llama_decode_step(llama_model *m, const int32_t *tokens, int32_t B, int32_t pos,
                               float *logits, int32_t *next_tokens, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): llama_decode_step with its scratch
 * (split-K sums of the few-row projections, decode-attention split partials, argmax
 * partials and, when logits is NULL, the step's logits) taken from a static array of
 * 64 MiB inside the library, one per GPU, held until the process ends, instead of the
 * model's workspace.  The results equal llama_decode_step's bit for bit.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (two streams, or two models)
 * race and must be serialised by the caller.  Nothing in the array needs clearing
 * between calls.  Errors as llama_decode_step, plus CAPACITY when the step needs more than
 * the 64 MiB (about B * (vocab * 4 + n_heads * (head_dim + 2) * 4 * ceil(max_seq / 256))
 * bytes). */
llama_status llama_decode_step_noalloc(llama_model *m, const int32_t *tokens, int32_t B,
                                       int32_t pos, float *logits, int32_t *next_tokens,
                                       hipStream_t stream);

/* Decode step of a ragged batch: sequence b's token tokens[b] sits at its own position
 * positions[b] (device memory, int32 [B]); its key and value are written at that position
 * and it attends to its cache positions 0..positions[b] (so sequences of different lengths
 * decode together; cache entries past a sequence's position are ignored).  Otherwise as
 * llama_decode_step.  positions is read on the device: a value outside [0, max_seq) makes
 * llama_sync_status report INVALID_ARG; that sequence's cache is left untouched and its
 * outputs are unspecified, and no access leaves the buffers. */
llama_status llama_decode_step_ragged(llama_model *m, const int32_t *tokens, int32_t B,
                                      const int32_t *positions, float *logits,
                                      int32_t *next_tokens, hipStream_t stream);

/* n_steps greedy decode steps starting with tokens[b] at position pos: step k runs at
 * position pos+k on the previous step's argmax (the article's greedy choice, section
 * 预测下一个输出, fed back as the next token over the pre-allocated cache of the Hacker
 * News thread).  The position and step index live in
 * device memory, so the whole loop is enqueued at once with no host synchronisation.
 * Writes out_tokens[k*B + b], the argmax of step k; if logits is not NULL also the logits
 * [n_steps,B,V].  Needs pos + n_steps <= max_seq.
 *
 * Stream capture: after the model's first call (its one-time set-up: flags, rotary table,
 * cache zero fill), llama_generate, llama_decode_step and llama_decode_step_ragged enqueue
 * kernel launches only (no memset, allocation or host synchronisation), so they may be
 * recorded into a stream capture and the graph replayed.  A replay repeats the recorded
 * arguments: the same start position for llama_generate and llama_decode_step, the
 * positions then in device memory for llama_decode_step_ragged. */
llama_status llama_generate(llama_model *m, const int32_t *tokens, int32_t B, int32_t pos,
                            int32_t n_steps, int32_t *out_tokens, float *logits,
                            hipStream_t stream);

/* One decoder layer on hidden states x_in [B,S,D] (fp32) of B sequences whose S tokens sit
 * at positions start_pos..start_pos+S-1; writes x_out [B,S,D] (may equal x_in) and the
 * layer's KV cache at those positions, attending to cache positions 0..start_pos+S-1.
 * With start_pos > 0 the cache must hold positions 0..start_pos-1 (chunked prefill). */
llama_status llama_layer_forward(llama_model *m, int32_t layer, const float *x_in,
                                 float *x_out, int32_t B, int32_t S, int32_t start_pos,
                                 hipStream_t stream);

/* Synchronise the stream, then report device-detected input errors since the last check
 * (token ids outside [0,V) give INVALID_ARG; their embedding rows are zero; NaN logits in
 * argmax give INVALID_ARG; so do ragged-decode positions outside [0, max_seq)) and clear
 * them.  The checks guard the embedding lookup (article, section 分词器与编码) and the
 * greedy argmax (section 预测下一个输出), whose inputs the host never sees. */
llama_status llama_sync_status(llama_model *m, hipStream_t stream);

/* Record the residual stream between the article's layers (section 预测下一个输出: the
 * embedding passes through the 32 layers in turn, then the final norm): while hidden is
 * set, each llama_prefill / llama_prefill_at / llama_decode_step(_ragged, _noalloc) /
 * llama_generate call writes, as fp32 rows of dim values, the input of every layer l to
 * hidden[l][row] (rows = B*S in token order for prefill, B for decode; after the
 * embedding for l = 0) and the rows the final RMSNorm reads to hidden[n_layers][row] (each
 * sequence's last position, or every position with all_positions; B rows in decode).
 * hidden holds (n_layers + 1) * max_rows * dim floats, 16-byte aligned, owned by the
 * caller; a call with more rows than max_rows returns CAPACITY.  llama_generate leaves its
 * last step.  llama_layer_forward is not recorded.  NULL stops recording.  Errors:
 * INVALID_ARG, SHAPE (max_rows <= 0). */
llama_status llama_trace_hidden(llama_model *m, float *hidden, int32_t max_rows);

/* Kernel classes of the forward pass, for llama_profile_kernel. */
typedef enum {
    LLAMA_KERNEL_NONE = 0,
    LLAMA_KERNEL_QKV = 1,        /* Q/K/V projection with RoPE and cache write        */
    LLAMA_KERNEL_ATTENTION = 2,  /* causal GQA attention (prefill or decode)           */
    LLAMA_KERNEL_WO = 3,         /* output projection with residual add (or split-K
                                    sums that the next RMSNorm adds)                  */
    LLAMA_KERNEL_FFN_UP = 4,     /* W1/W3 projection with SiLU * up                   */
    LLAMA_KERNEL_FFN_DOWN = 5,   /* W2 projection with residual add (or split-K sums
                                    that the next RMSNorm adds)                       */
    LLAMA_KERNEL_LM_HEAD = 6,    /* vocabulary projection                              */
    LLAMA_KERNEL_RMSNORM = 7     /* RMSNorm                                            */
} llama_kernel;

/* Start timing every launch of one kernel class with HIP events recorded on the call's
 * stream around it (LLAMA_KERNEL_NONE stops).  Launches recorded into a stream capture are
 * not timed.  Errors: INVALID_ARG. */
llama_status llama_profile_kernel(llama_model *m, llama_kernel kind);

/* Synchronise on the recorded events and report the summed duration in milliseconds and
 * the number of timed launches since llama_profile_kernel, then reset the counts. */
llama_status llama_profile_read(llama_model *m, double *total_ms, int32_t *launches);

/* Release the handle (the caller's buffers are untouched).  NULL is a no-op. */
void llama_free(llama_model *m);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *llama_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LLAMA_MI355X_H */
