"""GPU parity of the 8B-shaped stack at its full depth of 32 layers, through the C ABI.

Two kinds of check:

* Per layer with shared inputs.  The library records the residual stream of a real prefill
  or decode call (llama_trace_hidden): the input of every layer and the rows the final norm
  reads.  The float32 oracle runs each layer on the GPU's own input (for decode also over
  the GPU's own cache) and must land within the stated 2e-2 of the GPU's output of that
  layer; the head is checked the same way.  This measures one layer's kernel error at a
  time at the full shape, where a whole-stack comparison would mostly measure how the bf16
  recipe's rounding grows over 32 layers.
* End to end.  The GPU logits against the float32 oracle's own 32-layer chain, within
  max(2e-2, 1.5 x the gap the oracle's bf16 storage-point emulation shows on the same
  inputs), the bound derived for full depth; and the fp32 debug instantiation at the full
  8B shape within 1e-4 of a float64 oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import binding as bd
from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

from gpu_util import (BF16_TOL, F32_TOL, assert_rows_close, build_model, check_argmax,
                      require_gpu, rowwise_rel, say)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class _LayerCache:
    """The oracle's cache for one layer (index `layer`), pre-filled by the caller."""

    def __init__(self, layer, k, v):
        self.k = {layer: k}
        self.v = {layer: v}


def _layer_weights(synth, layer, dtype=np.float32):
    return {n: synth.as_float(n, dtype) for n, *_ in syn.layer_weight_specs(synth.spec, layer)}


def _head_weights(synth, dtype=np.float32):
    return {n: synth.as_float(n, dtype) for n in ("norm.weight", "output.weight")}


def test_prefill_2048_tokens_32_layers():
    """The 8B stack, 1 x 2048 tokens, 32 layers: the headline prefill."""
    spec = syn.LLAMA3_8B
    S, L = 2048, spec.n_layers
    say(f"8B, {L} layers: prefill 1 x {S} with the residual stream recorded")
    m, synth = build_model(spec, 3, max_batch=1, max_seq=S, max_tokens=S, cache=False)
    toks = syn.tokens(3, 1, S, spec.vocab_size)
    tdev = torch.from_numpy(toks).cuda()
    tr = m.trace_hidden(S)
    m.prefill(tdev, all_positions=True)
    hid = tr.cpu().numpy()                                   # [L + 1, S, D]
    m.trace_hidden(None)
    del tr
    # the benchmark's call: last-token logits and the greedy choice
    last, nxt = m.prefill(tdev, want_next=True)
    last = last.cpu().numpy()[0]
    nxt = int(nxt.cpu().numpy()[0])
    assert nxt == int(np.argmax(last))

    E = synth.as_float("tok_embeddings.weight", np.float32)
    np.testing.assert_array_equal(hid[0], E[toks[0]])        # the gather is exact
    x_ref = E[toks[0]].copy()
    x_emu = x_ref.copy()
    del E
    cap = S
    G, d = spec.n_kv_heads, spec.head_dim
    worst = 0.0
    for l in range(L):
        W = _layer_weights(synth, l)
        # llama_layer_forward on the recorded input reproduces the prefill's layer exactly
        x_gpu = m.layer_forward(l, torch.from_numpy(hid[l][None]).cuda()).cpu().numpy()[0]
        np.testing.assert_array_equal(x_gpu, hid[l + 1], err_msg=f"layer_forward, layer {l}")
        # shared input: the oracle's layer on the GPU's input of this layer
        c = _LayerCache(l, np.zeros((G, cap, d), np.float32), np.zeros((G, cap, d), np.float32))
        ref = O.layer_forward(hid[l], W, spec, l, c, 0)
        err = assert_rows_close(hid[l + 1], ref, BF16_TOL, f"layer {l} on shared input")
        worst = max(worst, float(err.max()))
        # the oracle's own chains, float32 and bf16 storage-point emulation
        c = _LayerCache(l, np.zeros((G, cap, d), np.float32), np.zeros((G, cap, d), np.float32))
        x_ref = O.layer_forward(x_ref, W, spec, l, c, 0)
        c = _LayerCache(l, np.zeros((G, cap, d), np.float32), np.zeros((G, cap, d), np.float32))
        x_emu = O.layer_forward(x_emu, W, spec, l, c, 0, bf16_points=True)
        del W, c
        if l % 8 == 7:
            say(f"  layers 0..{l}: worst shared-input error {worst:.3e}")
    Wh = _head_weights(synth)
    head_shared = O.head_logits(hid[L][-1:], Wh, spec)       # the last position [1, V]
    del hid
    assert_rows_close(last[None], head_shared, BF16_TOL, "head on the shared final row")
    check_argmax([nxt], last[None], head_shared, "greedy token, shared final row")
    full_ref = O.head_logits(x_ref[-1:], Wh, spec)
    full_emu = O.head_logits(x_emu[-1:], Wh, spec, bf16_points=True)
    gap = float(rowwise_rel(full_emu, full_ref).max())
    tol = max(BF16_TOL, 1.5 * gap)
    err = float(rowwise_rel(last[None], full_ref).max())
    say(f"  end to end, last-token logits: GPU vs float32 oracle {err:.3e}; bf16 emulation "
        f"vs float32 {gap:.3e}; bound {tol:.3e}; worst per-layer error {worst:.3e}")
    assert err <= tol, f"end-to-end error {err:.3e} above the bound {tol:.3e}"
    m.sync_status()


def test_fp32_debug_path_full_8b_shape():
    """The fp32 instantiation at the full 8B shape, 32 layers: prefill of 2 x 64 tokens at
    every position and two teacher-forced decode steps, row 0 within 1e-4 of a float64
    oracle."""
    spec = dataclasses.replace(syn.LLAMA3_8B, dtype="f32")
    B, S, steps = 2, 64, 2
    say(f"8B fp32 debug path, {spec.n_layers} layers: prefill {B} x {S}, {steps} decode steps")
    synth = syn.SyntheticWeights(spec, 30, cache=True)        # float32 draws, kept on the host
    w = bd.upload_weights(synth)
    m = bd.Model(spec, w, max_batch=B, max_seq=S + steps, max_tokens=B * S)
    toks = syn.tokens(30, B, S, spec.vocab_size)
    got, nxt0 = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True, want_next=True)
    got = got.cpu().numpy()
    nxt0 = nxt0.cpu().numpy()
    say("  oracle float64, row 0")
    W = syn.FloatView(synth, np.float64)
    ref, caches = O.prefill(toks[:1], W, spec, capacity=S + steps, all_positions=True,
                            dtype=np.float64)
    assert_rows_close(got[0], ref[0], F32_TOL, "prefill logits, every position")
    np.testing.assert_array_equal(nxt0, np.argmax(got[:, -1], axis=-1))
    check_argmax(nxt0[:1], got[:1, -1], ref[:, -1], "prefill greedy token")
    cur_ref = O.argmax(ref[:, -1]).astype(np.int32)
    cur = nxt0.astype(np.int32)
    for k in range(steps):
        cur[0] = cur_ref[0]
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        nxt = nxt.cpu().numpy()
        r = O.decode_step(cur_ref, S + k, W, spec, caches, dtype=np.float64)
        assert_rows_close(lg[:1], r, F32_TOL, f"decode step {k}")
        np.testing.assert_array_equal(nxt, np.argmax(lg, axis=-1))
        check_argmax(nxt[:1], lg[:1], r, f"decode step {k}")
        cur_ref = O.argmax(r).astype(np.int32)
        cur = nxt.astype(np.int32)
    m.sync_status()
    m.free()
    del m, w
    torch.cuda.empty_cache()


def test_decode_batch32_context4096_32_layers():
    """The decode headline's shape, 32 layers: batch 32 over 4096 prefilled positions, two
    greedy steps, rows 0 and 31 checked layer by layer on the GPU's own inputs and cache."""
    spec = syn.LLAMA3_8B
    B, ctx, steps, L = 32, 4096, 2, spec.n_layers
    rows = (0, 31)
    say(f"8B, {L} layers: prefill {B} x {ctx}, {steps} decode steps with the stream recorded")
    m, synth = build_model(spec, 4, max_batch=B, max_seq=ctx + steps, max_tokens=B * ctx,
                           cache=False)
    toks = syn.tokens(4, B, ctx, spec.vocab_size)
    _, cur = m.prefill(torch.from_numpy(toks).cuda(), want_next=True)
    tr = m.trace_hidden(B)
    hid, lgs, nxts = [], [], []
    for k in range(steps):
        nxt, lg = m.decode_step(cur, ctx + k)
        hid.append(tr.cpu().numpy()[:, list(rows)])           # [L + 1, rows, D]
        lgs.append(lg.cpu().numpy())
        nxts.append(nxt.cpu().numpy())
        np.testing.assert_array_equal(nxts[-1], np.argmax(lgs[-1], axis=-1))
        cur = nxt
    m.trace_hidden(None)
    worst = 0.0
    for l in range(L):
        W = _layer_weights(synth, l)
        for i, b in enumerate(rows):
            kc = m.cache_k(l)[b, :, :ctx + steps].float().cpu().numpy()
            vc = m.cache_v(l)[b, :, :ctx + steps].float().cpu().numpy()
            for k in range(steps):
                p = ctx + k
                # the oracle's cache for this layer: the GPU's keys and values at 0..p-1
                c = _LayerCache(l, kc[:, :p + 1].copy(), vc[:, :p + 1].copy())
                c.k[l][:, p] = 0.0
                c.v[l][:, p] = 0.0
                out = O.layer_forward(hid[k][l][i:i + 1], W, spec, l, c, p)
                err = assert_rows_close(hid[k][l + 1][i:i + 1], out, BF16_TOL,
                                        f"layer {l}, row {b}, step {k}")
                worst = max(worst, float(err.max()))
                # the key and value the GPU wrote at p
                assert_rows_close(kc[:, p].reshape(1, -1), c.k[l][:, p].reshape(1, -1), BF16_TOL,
                                  f"K written at {p}, layer {l}, row {b}")
                assert_rows_close(vc[:, p].reshape(1, -1), c.v[l][:, p].reshape(1, -1), BF16_TOL,
                                  f"V written at {p}, layer {l}, row {b}")
        del W
        if l % 8 == 7:
            say(f"  layers 0..{l}: worst shared-input error {worst:.3e}")
    Wh = _head_weights(synth)
    for k in range(steps):
        ref = O.head_logits(hid[k][L], Wh, spec)
        got = lgs[k][list(rows)]
        assert_rows_close(got, ref, BF16_TOL, f"head, step {k}")
        check_argmax(nxts[k][list(rows)], got, ref, f"greedy tokens, step {k}")
    say(f"  worst per-layer error {worst:.3e}")
    m.sync_status()


def test_long_context_4x8192_32_layers():
    """The long-context config at its full depth: 4 x 8192 tokens prefilled in one call, then
    two greedy steps of the batch.  The residual stream of the prefill is recorded; for every
    layer, sampled positions of sequences 0 and 3 run through the oracle's layer on the GPU's
    own input row and the GPU's own cache of the earlier positions (a position depends on
    nothing later), within 2e-2 of the GPU's output row, and the key and value the GPU wrote
    there are checked too; likewise rows 0 and 3 of both decode steps, and the head."""
    spec = syn.LLAMA3_8B
    B, S, steps, L = 4, 8192, 2, spec.n_layers
    seqs = (0, 3)
    rng = np.random.default_rng(5)
    pos = sorted(set([0, 1, 63, 64, 65, 2047, 4096, S - 2, S - 1] +
                     [int(p) for p in rng.integers(2, S - 2, 3)]))
    say(f"8B, {L} layers: prefill {B} x {S}, {steps} decode steps; positions {pos} of "
        f"sequences {seqs} checked per layer")
    m, synth = build_model(spec, 5, max_batch=B, max_seq=S + steps, max_tokens=B * S, cache=False)
    toks = syn.tokens(5, B, S, spec.vocab_size)
    # logits at every position, so that the final norm reads (and the trace records) the
    # last layer's output at every sampled position
    tr = m.trace_hidden(B * S)
    logits, cur = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True, want_next=True)
    rows = [b * S + p for b in seqs for p in pos]
    hid_p = tr[:, rows].cpu().numpy()                        # [L + 1, rows, D]
    m.trace_hidden(None)
    del tr
    lg_p = logits[list(seqs)][:, pos].cpu().numpy().reshape(len(rows), -1)
    last = logits[:, -1].cpu().numpy()
    del logits
    torch.cuda.empty_cache()
    cur_np = cur.cpu().numpy()
    np.testing.assert_array_equal(cur_np, np.argmax(last, axis=-1))
    # decode: two greedy steps with the stream of the batch recorded
    tr = m.trace_hidden(B)
    hid_d, lgs, nxts = [], [], []
    for k in range(steps):
        nxt, lg = m.decode_step(cur, S + k)
        hid_d.append(tr.cpu().numpy()[:, list(seqs)])
        lgs.append(lg.cpu().numpy())
        nxts.append(nxt.cpu().numpy())
        np.testing.assert_array_equal(nxts[-1], np.argmax(lgs[-1], axis=-1))
        cur = nxt
    m.trace_hidden(None)

    G, d = spec.n_kv_heads, spec.head_dim
    worst = 0.0
    for l in range(L):
        W = _layer_weights(synth, l)
        for i, b in enumerate(seqs):
            kc = m.cache_k(l)[b, :, :S + steps].float().cpu().numpy()
            vc = m.cache_v(l)[b, :, :S + steps].float().cpu().numpy()
            # prefill rows
            for j, p in enumerate(pos):
                r = i * len(pos) + j
                c = _LayerCache(l, kc[:, :p + 1].copy(), vc[:, :p + 1].copy())
                c.k[l][:, p] = 0.0
                c.v[l][:, p] = 0.0
                out = O.layer_forward(hid_p[l][r:r + 1], W, spec, l, c, p)
                err = assert_rows_close(hid_p[l + 1][r:r + 1], out, BF16_TOL,
                                        f"layer {l}, sequence {b}, position {p}")
                worst = max(worst, float(err.max()))
                assert_rows_close(kc[:, p].reshape(1, -1), c.k[l][:, p].reshape(1, -1), BF16_TOL,
                                  f"K at {p}, layer {l}, sequence {b}")
                assert_rows_close(vc[:, p].reshape(1, -1), c.v[l][:, p].reshape(1, -1), BF16_TOL,
                                  f"V at {p}, layer {l}, sequence {b}")
            # decode rows
            for k in range(steps):
                p = S + k
                c = _LayerCache(l, kc[:, :p + 1].copy(), vc[:, :p + 1].copy())
                c.k[l][:, p] = 0.0
                c.v[l][:, p] = 0.0
                out = O.layer_forward(hid_d[k][l][i:i + 1], W, spec, l, c, p)
                err = assert_rows_close(hid_d[k][l + 1][i:i + 1], out, BF16_TOL,
                                        f"decode step {k}, layer {l}, sequence {b}")
                worst = max(worst, float(err.max()))
                assert_rows_close(kc[:, p].reshape(1, -1), c.k[l][:, p].reshape(1, -1), BF16_TOL,
                                  f"K at {p}, layer {l}, sequence {b}")
        del W
        if l % 8 == 7:
            say(f"  layers 0..{l}: worst shared-input error {worst:.3e}")
    Wh = _head_weights(synth)
    ref = O.head_logits(hid_p[L], Wh, spec)
    assert_rows_close(lg_p, ref, BF16_TOL, "prefill head, sampled positions")
    lastr = [i * len(pos) + len(pos) - 1 for i in range(len(seqs))]   # position S - 1
    check_argmax(cur_np[list(seqs)], lg_p[lastr], ref[lastr], "prefill greedy tokens")
    for k in range(steps):
        ref = O.head_logits(hid_d[k][L], Wh, spec)
        got = lgs[k][list(seqs)]
        assert_rows_close(got, ref, BF16_TOL, f"decode head, step {k}")
        check_argmax(nxts[k][list(seqs)], got, ref, f"decode greedy tokens, step {k}")
    say(f"  worst per-layer error {worst:.3e}")
    m.sync_status()
