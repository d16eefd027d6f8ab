"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: values printed in the
article "250 lines of code to build Llama 3 from scratch" (ai02.cc), closed forms,
invariants, hand-computed tiny cases, or independent library routines (torch on the CPU).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ hyper-parameters

def test_ffn_hidden_size_of_llama3_8b_constants():
    # params.json constants (article, section 下载并读取模型权重): dim 4096, multiple_of 1024,
    # ffn_dim_multiplier 1.3.  2/3*4*4096 = 10922 -> *1.3 = 14198 -> up to 1024s = 14336.
    assert O.ffn_hidden_size(4096, 1024, 1.3) == 14336
    assert syn.LLAMA3_8B.ffn_hidden == 14336
    # rounding down instead of up would give 13312; no multiplier would give 11264
    assert O.ffn_hidden_size(4096, 1024, None) == 11264


def test_printed_weight_shapes():
    # article, section 查询向量: wq [4096,4096], wk [1024,4096], wv [1024,4096], wo [4096,4096];
    # section 预测下一个输出: output.weight [128256, 4096]; head_dim = 4096/32 = 128.
    shapes = {n: s for n, s, _, _ in syn.weight_specs(syn.LLAMA3_8B_ONE_LAYER)}
    assert shapes["layers.0.attention.wq.weight"] == (4096, 4096)
    assert shapes["layers.0.attention.wk.weight"] == (1024, 4096)
    assert shapes["layers.0.attention.wv.weight"] == (1024, 4096)
    assert shapes["layers.0.attention.wo.weight"] == (4096, 4096)
    assert shapes["output.weight"] == (128256, 4096)
    assert syn.LLAMA3_8B.dim // syn.LLAMA3_8B.n_heads == syn.LLAMA3_8B.head_dim == 128


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_unit_rms_closed_form():
    # Before the weight scale, y = x / sqrt(ms + eps) has RMS sqrt(ms / (ms + eps)).
    # Small-magnitude rows make eps matter, so a dropped or misplaced eps fails.
    rng = _rng(1)
    eps = 1e-5
    for scale in (1e-3, 1.0, 30.0):
        x = rng.standard_normal((7, 64)) * scale
        w = 1.0 + 0.1 * rng.standard_normal(64)
        y = O.rms_norm(x, w, eps)
        ms = np.mean(x * x, axis=-1)
        rms_unscaled = np.sqrt(np.mean((y / w) ** 2, axis=-1))
        np.testing.assert_allclose(rms_unscaled, np.sqrt(ms / (ms + eps)), rtol=1e-12)
        # direction of every row is kept, channel by channel through the weight
        np.testing.assert_allclose(y / w * np.sqrt(ms + eps)[:, None], x, rtol=1e-12, atol=1e-300)


def test_rmsnorm_matches_torch_library():
    rng = _rng(2)
    x = rng.standard_normal((5, 4096))
    w = 1.0 + 0.1 * rng.standard_normal(4096)
    ref = F.rms_norm(torch.from_numpy(x), (4096,), torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-5), ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ RoPE

def _golden_rope():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "rope_freqs_llama3_8b.txt"))
            if not l.startswith("#")]
    return (np.array([int(r[0]) for r in rows]), np.array([float(r[1]) for r in rows]),
            np.array([float(r[2]) for r in rows]))


def test_rope_frequencies_match_printed_table():
    i, exponents, freqs = _golden_rope()
    assert len(freqs) == 64
    theta_i = O.rope_frequencies(128, 500000.0)
    # printed to 5 significant figures: half a unit in the last place is <= 5e-5 relative
    np.testing.assert_allclose(theta_i, freqs, rtol=6e-5)
    # the exponents i/64 printed to 4 decimals
    np.testing.assert_allclose(-np.log(theta_i) / np.log(500000.0), exponents, atol=5.01e-5)


def test_rope_adjacent_pair_basis_vectors():
    # A unit vector in channel 2i at position m rotates to (cos m*theta_i, sin m*theta_i) in
    # channels (2i, 2i+1); one in channel 2i+1 goes to (-sin, cos).  Catches the half-split
    # pairing, a sign error and a wrong frequency index.
    d, theta = 16, 500000.0
    freqs = theta ** (-np.arange(d // 2) * 2.0 / d)
    for m in (0, 1, 7, 23):
        for i in range(d // 2):
            for which, expect in ((0, (math.cos(m * freqs[i]), math.sin(m * freqs[i]))),
                                  (1, (-math.sin(m * freqs[i]), math.cos(m * freqs[i])))):
                x = np.zeros((1, 1, d))
                x[0, 0, 2 * i + which] = 1.0
                y = O.rope_rotate(x, np.array([m]), theta)[0, 0]
                e = np.zeros(d)
                e[2 * i], e[2 * i + 1] = expect
                np.testing.assert_allclose(y, e, atol=1e-15)


def test_rope_matches_complex_form():
    # The article's form: view pairs as complex numbers, multiply by polar(1, m*theta_i).
    rng = _rng(3)
    S, nh, d = 9, 3, 128
    x = rng.standard_normal((S, nh, d))
    pos = np.arange(100, 100 + S)
    xc = x.reshape(S, nh, d // 2, 2)
    z = xc[..., 0] + 1j * xc[..., 1]
    i, _, _ = _golden_rope()
    ang = np.outer(pos, 500000.0 ** (-i / 64.0))
    zr = z * np.exp(1j * ang)[:, None, :]
    ref = np.stack([zr.real, zr.imag], axis=-1).reshape(S, nh, d)
    np.testing.assert_allclose(O.rope_rotate(x, pos, 500000.0), ref, rtol=1e-12, atol=1e-12)


def test_rope_preserves_norm_and_identity_at_zero():
    rng = _rng(4)
    x = rng.standard_normal((5, 2, 128))
    y = O.rope_rotate(x, np.array([0, 1, 50, 4095, 8255]), 500000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(O.rope_rotate(x[:1], np.array([0]), 500000.0), x[:1])


def test_rope_scores_depend_only_on_relative_position():
    rng = _rng(5)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for m, n in ((3, 1), (17, 17), (2000, 5)):
        base = np.sum(O.rope_rotate(q, [m], 5e5) * O.rope_rotate(k, [n], 5e5))
        for s in (1, 100, 6000):
            shifted = np.sum(O.rope_rotate(q, [m + s], 5e5) * O.rope_rotate(k, [n + s], 5e5))
            assert abs(shifted - base) <= 1e-11 * (1 + abs(base))


# ------------------------------------------------------------------ attention

def _sdpa_reference(q, k, v):
    # torch's scaled_dot_product_attention with K/V repeated per query group
    # (query head h uses KV head h // (H/G)); float64 on the CPU.
    S, H, d = q.shape
    G = k.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]              # [1,H,S,d]
    kt = torch.from_numpy(k).repeat_interleave(H // G, dim=0)[None]  # [1,H,S,d]
    vt = torch.from_numpy(v).repeat_interleave(H // G, dim=0)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("H,G", [(4, 2), (32, 8), (4, 4), (8, 1)])
def test_gqa_matches_torch_sdpa(H, G):
    rng = _rng(6)
    S, d = 19, 16
    q = rng.standard_normal((S, H, d))
    k = rng.standard_normal((G, S, d))
    v = rng.standard_normal((G, S, d))
    got = O.causal_gqa_attention(q, k, v, np.arange(S))
    np.testing.assert_allclose(got, _sdpa_reference(q, k, v), rtol=1e-11, atol=1e-12)


def test_position_zero_attends_only_to_itself():
    rng = _rng(7)
    S, H, G, d = 6, 4, 2, 8
    q = rng.standard_normal((S, H, d)) * 5
    k = rng.standard_normal((G, S, d)) * 5
    v = rng.standard_normal((G, S, d))
    out = O.causal_gqa_attention(q, k, v, np.arange(S))
    for h in range(H):
        np.testing.assert_array_equal(out[0, h], v[h // 2, 0])


def test_two_keys_by_hand():
    # One query at position 1 over two keys: softmax of two scaled scores.
    d = 4
    q = np.array([[[1.0, 2.0, 0.0, -1.0]]])
    k = np.array([[[0.5, 0.0, 1.0, 0.0], [1.0, 1.0, 1.0, 1.0]]])
    v = np.array([[[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 3.0]]])
    s0 = 0.5 / 2.0   # q.k0 / sqrt(4)
    s1 = 2.0 / 2.0   # q.k1 / sqrt(4)
    p1 = math.exp(s1) / (math.exp(s0) + math.exp(s1))
    out = O.causal_gqa_attention(q, k, v, np.array([1]))
    np.testing.assert_allclose(out[0, 0], [1 - p1, 0, 0, 3 * p1], rtol=1e-14)
    # at position 0 only the first key is visible
    out0 = O.causal_gqa_attention(q, k, v, np.array([0]))
    np.testing.assert_array_equal(out0[0, 0], v[0, 0])


def test_softmax_rows_and_masked_zeros():
    rng = _rng(8)
    s = rng.standard_normal((5, 5)) * 10
    s[np.triu_indices(5, 1)] = -np.inf
    p = O.softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-15)
    assert np.all(p[np.triu_indices(5, 1)] == 0.0)
    np.testing.assert_allclose(O.softmax(s + 123.0), p, rtol=1e-12)


# ------------------------------------------------------------------ feed-forward

def test_silu_matches_torch_library():
    z = np.linspace(-60, 60, 1001)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_swiglu_by_hand():
    # dim 2, hidden 1: gate = h.w1 = 1, up = h.w3 = 2, silu(1) = 1/(1+e^-1).
    h = np.array([[1.0, 2.0]])
    w1 = np.array([[1.0, 0.0]])
    w3 = np.array([[0.0, 1.0]])
    w2 = np.array([[1.0], [-1.0]])
    g = (1.0 / (1.0 + math.exp(-1.0))) * 2.0
    np.testing.assert_allclose(O.swiglu_ffn(h, w1, w3, w2), [[g, -g]], rtol=1e-15)


# ------------------------------------------------------------------ a whole layer

def _torch_layer(x, W, cfg, layer):
    """One decoder layer from torch library routines: rms_norm, complex RoPE (the
    article's polar/view_as_complex form), scaled_dot_product_attention, silu."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    p = f"layers.{layer}."
    S, D = x.shape
    H, G, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    xt = t(x)
    h = F.rms_norm(xt, (D,), t(W[p + "attention_norm.weight"]), eps=cfg.norm_eps)
    q = (h @ t(W[p + "attention.wq.weight"]).T).view(S, H, d)
    k = (h @ t(W[p + "attention.wk.weight"]).T).view(S, G, d)
    v = (h @ t(W[p + "attention.wv.weight"]).T).view(S, G, d)
    freqs = 1.0 / (cfg.rope_theta ** (torch.arange(d // 2, dtype=torch.float64) / (d // 2)))
    cis = torch.polar(torch.ones(S, d // 2, dtype=torch.float64),
                      torch.outer(torch.arange(S, dtype=torch.float64), freqs))
    rot = lambda a: torch.view_as_real(torch.view_as_complex(a.reshape(S, -1, d // 2, 2).contiguous())  # noqa: E731
                                       * cis[:, None, :]).reshape(S, -1, d)
    q, k = rot(q), rot(k)
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                       v.permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)
    xt = xt + o[0].permute(1, 0, 2).reshape(S, H * d) @ t(W[p + "attention.wo.weight"]).T
    h2 = F.rms_norm(xt, (D,), t(W[p + "ffn_norm.weight"]), eps=cfg.norm_eps)
    ff = (F.silu(h2 @ t(W[p + "feed_forward.w1.weight"]).T) * (h2 @ t(W[p + "feed_forward.w3.weight"]).T)) \
        @ t(W[p + "feed_forward.w2.weight"]).T
    return (xt + ff).numpy()


def test_layer_matches_torch_library_composition():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=1))
    x = syn.normal(1, "x", (17, cfg.dim)).astype(np.float64)
    cache = O.SequenceCache(cfg, 17)
    got = O.layer_forward(x, W, cfg, 0, cache, 0)
    np.testing.assert_allclose(got, _torch_layer(x, W, cfg, 0), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ the whole stack

def _torch_stack(tokens, W, cfg):
    """The stack from torch library routines (article, sections 分词器与编码 and
    预测下一个输出): F.embedding of tok_embeddings, the layers in order (each from
    _torch_layer), one F.rms_norm with norm.weight, then F.linear with output.weight.
    Logits of every position [S, V]."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    x = F.embedding(torch.from_numpy(np.asarray(tokens, dtype=np.int64)), t(W["tok_embeddings.weight"]))
    for layer in range(cfg.n_layers):
        x = torch.from_numpy(_torch_layer(x.numpy(), W, cfg, layer))
    y = F.rms_norm(x, (cfg.dim,), t(W["norm.weight"]), eps=cfg.norm_eps)
    return F.linear(y, t(W["output.weight"])).numpy()


def _stack_pin_holds(seed=12):
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=seed))
    toks = syn.tokens(seed, 1, 17, cfg.vocab_size)
    got, _ = O.prefill(toks, W, cfg, all_positions=True)
    last, _ = O.prefill(toks, W, cfg)
    ref = _torch_stack(toks[0], W, cfg)
    return (np.allclose(got[0], ref, rtol=1e-11, atol=1e-11)
            and np.allclose(last[0], ref[-1], rtol=1e-11, atol=1e-11))


def test_stack_matches_torch_library_composition():
    # embedding, the layer loop, the final norm applied once and the untied output
    # projection, each from an independent library routine
    assert _stack_pin_holds()


def test_embedding_rows_by_hand():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=13))
    toks = np.array([0, 255, 7, 7, 128])
    x = O.embed(toks, W)
    E = W["tok_embeddings.weight"]
    for i, tok in enumerate(toks):
        np.testing.assert_array_equal(x[i], E[tok])


def _planted(monkeypatch, which):
    """Plant one plausible mistake in the oracle (on the CPU) and report whether the stack
    pin still holds."""
    real_embed, real_head, real_layer = O.embed, O.head_logits, O.layer_forward
    if which == "final norm twice":
        def head(x, weights, cfg, bf16_points=False):
            w = np.asarray(weights["norm.weight"], dtype=x.dtype)
            y = O.rms_norm(O.rms_norm(x, w, cfg.norm_eps), w, cfg.norm_eps)
            return y @ np.asarray(weights["output.weight"], dtype=x.dtype).T
        monkeypatch.setattr(O, "head_logits", head)
    elif which == "head tied to the embedding":
        def head(x, weights, cfg, bf16_points=False):
            y = O.rms_norm(x, np.asarray(weights["norm.weight"], dtype=x.dtype), cfg.norm_eps)
            return y @ np.asarray(weights["tok_embeddings.weight"], dtype=x.dtype).T
        monkeypatch.setattr(O, "head_logits", head)
    elif which == "wrong embedding row":
        monkeypatch.setattr(O, "embed", lambda tokens, weights, dtype=np.float64:
                            real_embed((np.asarray(tokens) + 1) % 256, weights, dtype))
    elif which == "layers in reverse order":
        def layer(x, weights, cfg, layer, cache, start_pos, bf16_points=False):
            return real_layer(x, weights, cfg, cfg.n_layers - 1 - layer, cache, start_pos, bf16_points)
        monkeypatch.setattr(O, "layer_forward", layer)
    elif which == "no final norm":
        def head(x, weights, cfg, bf16_points=False):
            return x @ np.asarray(weights["output.weight"], dtype=x.dtype).T
        monkeypatch.setattr(O, "head_logits", head)
    elif which == "last layer skipped":
        def layer(x, weights, cfg, layer, cache, start_pos, bf16_points=False):
            if layer == cfg.n_layers - 1:
                return x
            return real_layer(x, weights, cfg, layer, cache, start_pos, bf16_points)
        monkeypatch.setattr(O, "layer_forward", layer)
    else:
        raise ValueError(which)
    try:
        return _stack_pin_holds()
    finally:
        monkeypatch.setattr(O, "embed", real_embed)
        monkeypatch.setattr(O, "head_logits", real_head)
        monkeypatch.setattr(O, "layer_forward", real_layer)


@pytest.mark.parametrize("mistake", ["final norm twice", "head tied to the embedding",
                                     "wrong embedding row", "layers in reverse order",
                                     "no final norm", "last layer skipped"])
def test_stack_pin_catches_planted_mistakes(monkeypatch, mistake):
    assert _stack_pin_holds()
    assert not _planted(monkeypatch, mistake), f"the stack pin missed: {mistake}"
    assert _stack_pin_holds()


# ------------------------------------------------------------------ cache and decode invariants

def test_decode_reproduces_prefill_logits():
    # Token-by-token decode over the cache gives the all-position prefill logits.
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=1))
    toks = syn.tokens(1, 1, 17, cfg.vocab_size)
    full, _ = O.prefill(toks, W, cfg, all_positions=True)
    cache = [O.SequenceCache(cfg, 17)]
    for pos in range(17):
        lg = O.decode_step(toks[:, pos], pos, W, cfg, cache)
        np.testing.assert_allclose(lg[0], full[0, pos], rtol=1e-12, atol=1e-12)


def test_chunked_prefill_equals_single_prefill():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=2))
    x = syn.normal(2, "x", (17, cfg.dim)).astype(np.float64)
    c1 = O.SequenceCache(cfg, 17)
    whole = O.layer_forward(x, W, cfg, 0, c1, 0)
    c2 = O.SequenceCache(cfg, 17)
    a = O.layer_forward(x[:5], W, cfg, 0, c2, 0)
    b = O.layer_forward(x[5:], W, cfg, 0, c2, 5)
    np.testing.assert_allclose(np.concatenate([a, b]), whole, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c2.k[0], c1.k[0], rtol=1e-12, atol=1e-13)


def test_prefill_in_chunks_equals_one_prefill():
    # prefill_sequence_at over the chunks [0,6), [6,11), [11,17) gives the all-position
    # logits of one prefill of the 17 tokens, and the same cache.
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=4))
    toks = syn.tokens(4, 1, 17, cfg.vocab_size)[0]
    full, caches = O.prefill(toks[None], W, cfg, all_positions=True)
    cache = O.SequenceCache(cfg, 17)
    parts = [O.prefill_sequence_at(toks[a:b], a, W, cfg, cache, all_positions=True)
             for a, b in ((0, 6), (6, 11), (11, 17))]
    np.testing.assert_allclose(np.concatenate(parts), full[0], rtol=1e-12, atol=1e-12)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(cache.v[l], caches[0].v[l], rtol=1e-12, atol=1e-13)
    last = O.prefill_sequence_at(toks[11:], 11, W, cfg, O.SequenceCache(cfg, 17))
    assert last.shape == (cfg.vocab_size,)


def test_ragged_decode_positions_reproduce_prefill():
    # Rows decoding at different positions over a cache filled further than their position
    # (the entries past it are ignored and overwritten) give the prefill logits there.
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=5))
    toks = syn.tokens(5, 3, 13, cfg.vocab_size)
    full, caches = O.prefill(toks, W, cfg, all_positions=True)
    for b, pos in enumerate((4, 12, 9)):
        lg = O.decode_sequence_step(int(toks[b, pos]), pos, W, cfg, caches[b])
        np.testing.assert_allclose(lg, full[b, pos], rtol=1e-12, atol=1e-12)


def test_batch_rows_are_independent():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=3))
    toks = syn.tokens(3, 3, 9, cfg.vocab_size)
    lg, _ = O.prefill(toks, W, cfg)
    for b in range(3):
        one, _ = O.prefill(toks[b:b + 1], W, cfg)
        np.testing.assert_array_equal(one[0], lg[b])


def test_greedy_generate_consistent_with_prefill():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=1))
    toks = syn.tokens(1, 1, 17, cfg.vocab_size)
    l0, ls, chosen = O.greedy_generate(toks, 4, W, cfg)
    assert chosen.shape == (5, 1) and ls.shape == (4, 1, cfg.vocab_size)
    # re-running the full sequence (prompt + chosen tokens) as one prefill gives the same logits
    seq = np.concatenate([toks, chosen[:-1].T], axis=1)
    full, _ = O.prefill(seq, W, cfg, all_positions=True)
    np.testing.assert_allclose(full[0, 16], l0[0], rtol=1e-12, atol=1e-12)
    for k in range(4):
        np.testing.assert_allclose(full[0, 17 + k], ls[k, 0], rtol=1e-12, atol=1e-12)


def test_argmax_lowest_index_on_ties():
    assert O.argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    np.testing.assert_array_equal(O.argmax(np.array([[0.0, 0.0], [-1.0, 5.0]])), [0, 1])
    with pytest.raises(ValueError):
        O.argmax(np.array([0.0, np.nan]))


def test_one_8b_layer_shapes_float32():
    # Article's shape checkpoints at 17 tokens: [17,4096] in and out, q per head [17,128],
    # cache per KV head [17,128] for 8 KV heads.
    cfg = syn.LLAMA3_8B_ONE_LAYER
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=2, cache=False), np.float32)
    x = syn.normal(2, "x", (17, 4096))
    cache = O.SequenceCache(cfg, 17, np.float32)
    y = O.layer_forward(x, W, cfg, 0, cache, 0)
    assert y.shape == (17, 4096) and y.dtype == np.float32
    assert cache.k[0].shape == (8, 17, 128) and cache.v[0].shape == (8, 17, 128)
    assert np.isfinite(y).all()


# ------------------------------------------------------------------ bf16 emulation (diagnostic)

def test_round_bf16_matches_torch_library():
    rng = _rng(9)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-8, 8, 10000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0])])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.round_bf16(x32), ref)
    np.testing.assert_array_equal(O.round_bf16(ref), ref)  # idempotent on bf16 values


def test_bf16_emulation_is_off_by_default_and_small():
    cfg = syn.TINY
    W = syn.FloatView(syn.SyntheticWeights(cfg, seed=1))
    toks = syn.tokens(1, 1, 17, cfg.vocab_size)
    a, _ = O.prefill(toks, W, cfg, all_positions=True)
    b, _ = O.prefill(toks, W, cfg, all_positions=True, bf16_points=False)
    c, _ = O.prefill(toks, W, cfg, all_positions=True, bf16_points=True)
    np.testing.assert_array_equal(a, b)
    rel = np.max(np.abs(c - a), -1) / np.max(np.abs(a), -1)
    assert 0 < rel.max() < 2e-2


# ------------------------------------------------------------------ synthetic recipe

def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], dtype=np.float32)
    got = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(vals))
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got, ref)


def test_synthetic_is_deterministic_and_thread_independent():
    a = syn.normal(5, "w", (3, 1 << 21), std=0.02, dtype="bf16", threads=1)
    b = syn.normal(5, "w", (3, 1 << 21), std=0.02, dtype="bf16", threads=4)
    np.testing.assert_array_equal(a, b)
    f = syn.bf16_bits_to_f32(a)
    assert abs(f.std() - 0.02) < 1e-4 and abs(f.mean()) < 1e-4
