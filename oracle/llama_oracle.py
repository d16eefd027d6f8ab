"""Plain CPU reference of the Llama-3 decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code with the GPU library: it imports numpy and nothing else.

Every function follows the article "250 lines of code to build Llama 3 from scratch"
(ai02.cc, a walk-through of naklecha/llama3-from-scratch); section names are the article's
headings.  RMSNorm is also given on the "Deepdive-llama3-from-scratch" page (pitchhut.com),
in its layer-normalisation example.  The KV cache is described only in words, on the Hacker
News thread "Llama 3 implemented in pure NumPy" (the cache is pre-allocated by
max_seq_len x max_batch_size) and on the pitchhut page (a KV-cache chapter); its contents
here are the plainest reading: post-RoPE keys and raw values of every position so far.

Arithmetic is done in the floating type the caller asks for (float64 by default, float32
for the large shapes).  Nothing is fused, blocked or reordered: projections are separate
matrix products, attention is an explicit loop over heads over the full masked score
matrix, as in the article's head loop.

Configuration objects are duck-typed: anything with the attributes ``dim, n_layers,
n_heads, n_kv_heads, head_dim, ffn_hidden, vocab_size, norm_eps, rope_theta``.

Weights are a mapping from the checkpoint key names (article, section 下载并读取模型权重)
to float arrays stored [out, in], used as ``x @ W.T``.

Parity pins: every function is pinned by tests that do not call it to check itself
(printed values, closed forms, library special cases, brute force); see tests/.

Optional bf16 storage-point emulation (``bf16_points=True``): the values a bf16 inference
path stores in bfloat16 (the normalised GEMM inputs, q, the cached k and v, the softmax
probabilities the article casts to bf16 in its head loop, the attention output, the
feed-forward hidden state) are rounded to bfloat16 where they are produced.  It is a
diagnostic used to size the expected gap between a bf16 path and this float reference;
it is never the reference itself.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------------------
# Hyper-parameters
# ---------------------------------------------------------------------------------------

def ffn_hidden_size(dim: int, multiple_of: int, ffn_dim_multiplier: float | None) -> int:
    """Hidden width of the SwiGLU feed-forward.

    The article prints only the constants (params.json in section 下载并读取模型权重:
    dim 4096, multiple_of 1024, ffn_dim_multiplier 1.3).  The rule used to turn them into a
    width is the one the Llama family uses: take 2/3 of 4*dim, scale by the multiplier,
    round up to a multiple of ``multiple_of``.
    """
    hidden = int(2 * (4 * dim) / 3)
    if ffn_dim_multiplier is not None:
        hidden = int(ffn_dim_multiplier * hidden)
    return multiple_of * ((hidden + multiple_of - 1) // multiple_of)


# ---------------------------------------------------------------------------------------
# bfloat16 rounding (diagnostic emulation only)
# ---------------------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even) and return it in x's float type.

    bfloat16 keeps the top 16 bits of a float32; rounding adds 0x7FFF plus the lowest kept
    bit before truncating.  Done on a float32 view; NaN/Inf are not expected here.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs: the sum stays below 2**32 (the largest finite bit pattern is 0x7F7FFFFF
    # or 0xFF7FFFFF, and at most 0x8000 is added)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.asarray(x).dtype)


def _maybe_bf16(x: np.ndarray, on: bool) -> np.ndarray:
    return round_bf16(x) if on else x


# ---------------------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------------------

def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x * 1/sqrt(mean(x^2) + eps), then times the per-channel weight; per token.

    Article, section 分词器与编码 (tokeniser and embedding) defines ``rms_norm`` this way,
    and the pitchhut page's layer-normalisation example repeats it.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x * (1.0 / np.sqrt(ms + eps))) * weight


# ---------------------------------------------------------------------------------------
# Rotary position embedding
# ---------------------------------------------------------------------------------------

def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """theta_i = theta ** (-i / (head_dim/2)) for i in [0, head_dim/2), in float64.

    Article, section 位置编码 (positional encoding): the exponents are range(64)/64 and the
    frequencies 1 / rope_theta ** exponent, at head_dim 128.
    """
    half = head_dim // 2
    exponents = np.arange(half, dtype=np.float64) / half
    return 1.0 / (float(theta) ** exponents)


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, dtype=np.float64):
    """cos and sin of the angle m * theta_i, [len(positions), head_dim/2].

    Article, section 位置编码: ``outer(positions, freqs)`` then ``polar(1, angle)``.  The
    angle is formed in float64 and its cosine and sine are rounded to ``dtype``.
    """
    angle = np.outer(np.asarray(positions, dtype=np.float64), rope_frequencies(head_dim, theta))
    return np.cos(angle).astype(dtype), np.sin(angle).astype(dtype)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate adjacent pairs (x[2i], x[2i+1]) of every head vector by the angle m * theta_i.

    ``x`` is [S, n_heads, head_dim] and ``positions`` gives m for each of the S rows.
    Article, section 位置编码: the vector is viewed as 64 pairs, each pair as one complex
    number, multiplied elementwise by polar(1, m * theta_i), and viewed back as reals.  The
    complex product written out in real arithmetic is
    (a + ib)(c + is) = (a c - b s) + i (a s + b c).
    """
    S, nh, d = x.shape
    c, s = rope_cos_sin(positions, d, theta, dtype=x.dtype)  # [S, d/2]
    pairs = x.reshape(S, nh, d // 2, 2)
    a = pairs[..., 0]
    b = pairs[..., 1]
    c = c[:, None, :]
    s = s[:, None, :]
    out = np.empty_like(pairs)
    out[..., 0] = a * c - b * s
    out[..., 1] = a * s + b * c
    return out.reshape(S, nh, d)


# ---------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------

def softmax(scores: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, with the row maximum subtracted first (exact in real
    arithmetic; keeps exp finite).  Masked entries are -inf and become exactly 0."""
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_gqa_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                         query_positions: np.ndarray, bf16_points: bool = False) -> np.ndarray:
    """Grouped-query causal attention for one sequence.

    q: [S, H, d] (rotated); keys, values: [G, ctx, d] (keys rotated), holding positions
    0..ctx-1.  Query head h reads KV head h // (H/G) (article, section 多头注意力: key and
    value weights are shared across 4 heads, ``head//4``).  Scores are q.k / sqrt(d)
    (section 查询和键相乘); key positions after the query's own position get -inf
    (section 多头注意力: ``triu(full(-inf), diagonal=1)``); softmax runs over the keys
    (``dim=1``); the output is softmax . v (section 注意力向量).  Returns [S, H, d].
    """
    S, H, d = q.shape
    G, ctx, _ = keys.shape
    group = H // G
    key_pos = np.arange(ctx)
    mask = np.where(key_pos[None, :] > np.asarray(query_positions)[:, None], -np.inf, 0.0)
    out = np.empty_like(q)
    for head in range(H):
        kv = head // group
        scores = (q[:, head, :] @ keys[kv].T) / math.sqrt(d)
        probs = _maybe_bf16(softmax(scores + mask), bf16_points)
        out[:, head, :] = probs @ values[kv]
    return out


# ---------------------------------------------------------------------------------------
# Feed-forward
# ---------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z)).  The article calls F.silu without defining it."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(h: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """(silu(h W1^T) * (h W3^T)) W2^T.  Article, section 前馈神经网络层 (feed-forward)."""
    return (silu(h @ w1.T) * (h @ w3.T)) @ w2.T


# ---------------------------------------------------------------------------------------
# One decoder layer over one sequence, with its cache
# ---------------------------------------------------------------------------------------

class SequenceCache:
    """Keys (rotated) and values of every position so far, per layer, for one sequence.

    Layer l holds ``k[l]``, ``v[l]``: [G, capacity, d].  The pre-allocated capacity follows
    the Hacker News thread's note that the cache is pre-allocated by max_seq_len.
    """

    def __init__(self, cfg, capacity: int, dtype=np.float64):
        G, d = cfg.n_kv_heads, cfg.head_dim
        self.k = [np.zeros((G, capacity, d), dtype=dtype) for _ in range(cfg.n_layers)]
        self.v = [np.zeros((G, capacity, d), dtype=dtype) for _ in range(cfg.n_layers)]


def layer_forward(x: np.ndarray, weights, cfg, layer: int, cache: SequenceCache,
                  start_pos: int, bf16_points: bool = False) -> np.ndarray:
    """One decoder layer for the S tokens of one sequence at positions start_pos..start_pos+S-1.

    Article, sections 构建Transformer层 through 前馈神经网络层, in order:
      h = rms_norm(x, attention_norm)
      q, k, v = h Wq^T, h Wk^T, h Wv^T, viewed per head (row = head*d + i)
      q, k rotated by position; k and v appended to the cache
      attention over cache positions 0..start_pos+S-1, causal
      x = x + concat(heads) Wo^T                      (section 相加与归一化)
      x = x + swiglu(rms_norm(x, ffn_norm))           (section 前馈神经网络层)
    """
    dt = x.dtype
    S, D = x.shape
    H, G, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    p = f"layers.{layer}."
    W = lambda name: np.asarray(weights[p + name], dtype=dt)  # noqa: E731

    positions = start_pos + np.arange(S)
    b16 = bf16_points
    h = _maybe_bf16(rms_norm(x, W("attention_norm.weight"), cfg.norm_eps), b16)
    q = (h @ W("attention.wq.weight").T).reshape(S, H, d)
    k = (h @ W("attention.wk.weight").T).reshape(S, G, d)
    v = _maybe_bf16((h @ W("attention.wv.weight").T).reshape(S, G, d), b16)
    q = _maybe_bf16(rope_rotate(q, positions, cfg.rope_theta), b16)
    k = _maybe_bf16(rope_rotate(k, positions, cfg.rope_theta), b16)

    cache.k[layer][:, start_pos:start_pos + S, :] = k.transpose(1, 0, 2)
    cache.v[layer][:, start_pos:start_pos + S, :] = v.transpose(1, 0, 2)
    ctx = start_pos + S
    attn = causal_gqa_attention(q, cache.k[layer][:, :ctx, :], cache.v[layer][:, :ctx, :],
                                positions, bf16_points=b16)

    x = x + _maybe_bf16(attn.reshape(S, H * d), b16) @ W("attention.wo.weight").T
    h2 = _maybe_bf16(rms_norm(x, W("ffn_norm.weight"), cfg.norm_eps), b16)
    if b16:
        g = round_bf16(silu(h2 @ W("feed_forward.w1.weight").T) * (h2 @ W("feed_forward.w3.weight").T))
        x = x + g @ W("feed_forward.w2.weight").T
    else:
        x = x + swiglu_ffn(h2, W("feed_forward.w1.weight"), W("feed_forward.w3.weight"),
                           W("feed_forward.w2.weight"))
    return x


# ---------------------------------------------------------------------------------------
# The whole stack
# ---------------------------------------------------------------------------------------

def embed(tokens: np.ndarray, weights, dtype=np.float64) -> np.ndarray:
    """Rows of tok_embeddings for each token id (article, section 分词器与编码)."""
    return np.asarray(weights["tok_embeddings.weight"], dtype=dtype)[np.asarray(tokens)]


def head_logits(x: np.ndarray, weights, cfg, bf16_points: bool = False) -> np.ndarray:
    """Final RMSNorm, applied once, then the output projection to vocabulary logits
    (article, section 预测下一个输出)."""
    y = rms_norm(x, np.asarray(weights["norm.weight"], dtype=x.dtype), cfg.norm_eps)
    y = _maybe_bf16(y, bf16_points)
    return y @ np.asarray(weights["output.weight"], dtype=x.dtype).T


def prefill_sequence(tokens: np.ndarray, weights, cfg, cache: SequenceCache,
                     all_positions: bool = False, dtype=np.float64,
                     bf16_points: bool = False) -> np.ndarray:
    """Causal prefill of one sequence from position 0.

    Returns the logits of the last position [V], or of every position [S, V]
    (article, section 预测下一个输出: the stack of layers, the final norm and
    ``final_embedding[-1] @ output.weight^T``).
    """
    x = embed(tokens, weights, dtype)
    for layer in range(cfg.n_layers):
        x = layer_forward(x, weights, cfg, layer, cache, start_pos=0, bf16_points=bf16_points)
    if all_positions:
        return head_logits(x, weights, cfg, bf16_points)
    return head_logits(x[-1:], weights, cfg, bf16_points)[0]


def prefill_sequence_at(tokens: np.ndarray, start_pos: int, weights, cfg, cache: SequenceCache,
                        all_positions: bool = False, dtype=np.float64) -> np.ndarray:
    """Continue one sequence with the tokens at positions start_pos..start_pos+S-1, the cache
    already holding positions 0..start_pos-1 (chunked prefill).  The same steps as
    prefill_sequence, with the layers run at those positions: each token attends to every
    cached position up to its own (article, section 多头注意力, the causal mask; the
    pre-allocated cache of the Hacker News thread).  Returns the logits of the last
    position [V], or of every new position [S, V]."""
    x = embed(tokens, weights, dtype)
    for layer in range(cfg.n_layers):
        x = layer_forward(x, weights, cfg, layer, cache, start_pos=start_pos)
    if all_positions:
        return head_logits(x, weights, cfg)
    return head_logits(x[-1:], weights, cfg)[0]


def decode_sequence_step(token: int, pos: int, weights, cfg, cache: SequenceCache,
                         dtype=np.float64) -> np.ndarray:
    """One KV-cache decode step: the single token at position ``pos`` attends to the cached
    positions 0..pos-1 and to itself; returns its logits [V]."""
    x = embed(np.array([token]), weights, dtype)
    for layer in range(cfg.n_layers):
        x = layer_forward(x, weights, cfg, layer, cache, start_pos=pos)
    return head_logits(x, weights, cfg)[0]


def argmax(logits: np.ndarray) -> np.ndarray:
    """Greedy choice over the last axis; the lowest index wins among equal maxima
    (article, section 预测下一个输出: ``torch.argmax``)."""
    logits = np.asarray(logits)
    if np.isnan(logits).any():
        raise ValueError("NaN logits")
    return np.argmax(logits, axis=-1)


def prefill(tokens: np.ndarray, weights, cfg, capacity: int | None = None,
            all_positions: bool = False, dtype=np.float64, bf16_points: bool = False):
    """Batch prefill: each row of ``tokens`` [B, S] is an independent sequence.

    Returns (logits [B, V] or [B, S, V], list of per-row caches)."""
    tokens = np.asarray(tokens)
    B, S = tokens.shape
    caches = [SequenceCache(cfg, capacity or S, dtype) for _ in range(B)]
    logits = np.stack([prefill_sequence(tokens[b], weights, cfg, caches[b], all_positions, dtype,
                                        bf16_points) for b in range(B)])
    return logits, caches


def decode_step(tokens: np.ndarray, pos: int, weights, cfg, caches, dtype=np.float64):
    """Batch decode step at position ``pos`` for every row; returns logits [B, V]."""
    return np.stack([decode_sequence_step(int(t), pos, weights, cfg, caches[b], dtype)
                     for b, t in enumerate(np.asarray(tokens))])


def greedy_generate(tokens: np.ndarray, steps: int, weights, cfg, dtype=np.float64):
    """Prefill, then ``steps`` greedy decode steps, each fed the previous argmax.

    Returns (prefill logits [B, V], decode logits [steps, B, V], chosen tokens
    [steps + 1, B]): the first chosen token comes from the prefill logits.
    """
    tokens = np.asarray(tokens)
    B, S = tokens.shape
    logits0, caches = prefill(tokens, weights, cfg, capacity=S + steps, dtype=dtype)
    chosen = [argmax(logits0)]
    step_logits = []
    for k in range(steps):
        lg = decode_step(chosen[-1], S + k, weights, cfg, caches, dtype)
        step_logits.append(lg)
        chosen.append(argmax(lg))
    return logits0, np.stack(step_logits) if steps else np.zeros((0, B, cfg.vocab_size)), np.stack(chosen)
