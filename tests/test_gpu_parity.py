"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Sizes here finish in seconds on the oracle and still span several GEMM / attention tiles
and a ragged tail.  bf16 results must be within 2e-2 normwise per row of the oracle
(float64, fed the exact bf16 weights); the fp32 debug path within 1e-4.
"""
import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import binding as bd
from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

from gpu_util import (BF16_TOL, F32_TOL, assert_rows_close, build_model, check_argmax,
                      require_gpu, say, small_bf16_spec)

# a hung GPU call ends the run (thread method) instead of stalling it
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ------------------------------------------------------------------ tiny fp32 stack

def test_tiny_fp32_prefill_all_positions():
    say("tiny fp32 prefill: B=1 S=17")
    spec = syn.TINY
    m, synth = build_model(spec, 1, max_batch=1, max_seq=32, max_tokens=32)
    toks = syn.tokens(1, 1, 17, spec.vocab_size)
    got = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    ref, _ = O.prefill(toks, syn.FloatView(synth), spec, all_positions=True)
    assert_rows_close(got, ref, F32_TOL, "tiny prefill logits")
    last = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    np.testing.assert_array_equal(last[0], got[0, -1])
    m.sync_status()


def test_tiny_fp32_greedy_decode_matches_oracle():
    say("tiny fp32: prefill + 8 greedy decode steps")
    spec = syn.TINY
    m, synth = build_model(spec, 1, max_batch=1, max_seq=32, max_tokens=32)
    toks = syn.tokens(1, 1, 17, spec.vocab_size)
    l0_ref, ls_ref, chosen_ref = O.greedy_generate(toks, 8, syn.FloatView(synth), spec)
    l0 = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    assert_rows_close(l0, l0_ref, F32_TOL, "prefill logits")
    cur = torch.tensor(np.argmax(l0, axis=-1).astype(np.int32)).cuda()
    chosen = [cur.cpu().numpy()]
    for k in range(8):
        nxt, lg = m.decode_step(cur, 17 + k)
        assert_rows_close(lg.cpu().numpy(), ls_ref[k], F32_TOL, f"decode step {k}")
        chosen.append(nxt.cpu().numpy())
        cur = nxt
    np.testing.assert_array_equal(np.stack(chosen), chosen_ref)   # strict at fp32
    m.sync_status()


def test_tiny_fp32_generate_loop_matches_oracle():
    say("tiny fp32: generate and generate with logits")
    spec = syn.TINY
    m, synth = build_model(spec, 1, max_batch=2, max_seq=40, max_tokens=40)
    toks = syn.tokens(1, 2, 17, spec.vocab_size)
    _, ls_ref, chosen_ref = O.greedy_generate(toks, 8, syn.FloatView(synth), spec)
    l0, first = m.prefill(torch.from_numpy(toks).cuda(), want_next=True)
    np.testing.assert_array_equal(first.cpu().numpy(), chosen_ref[0])
    out, _ = m.generate(first, 17, 8)
    np.testing.assert_array_equal(out.cpu().numpy(), chosen_ref[1:])
    # again with logits (eager steps), after re-prefilling the cache
    m.prefill(torch.from_numpy(toks).cuda())
    out2, lg = m.generate(first, 17, 8, want_logits=True)
    np.testing.assert_array_equal(out2.cpu().numpy(), chosen_ref[1:])
    assert_rows_close(lg.cpu().numpy(), ls_ref, F32_TOL, "generate logits")
    # a second generate run from the same cache gives the same tokens
    m.prefill(torch.from_numpy(toks).cuda())
    out3, _ = m.generate(first, 17, 8)
    np.testing.assert_array_equal(out3.cpu().numpy(), chosen_ref[1:])
    m.sync_status()


# ------------------------------------------------------------------ 8B-shaped layer, S=17

def test_llama3_8b_layer_bf16_seq17():
    say("8B-shaped layer bf16: B=1 S=17")
    spec = syn.LLAMA3_8B_ONE_LAYER
    m, synth = build_model(spec, 2, max_batch=1, max_seq=64, max_tokens=64)
    x = syn.normal(2, "x", (1, 17, spec.dim))
    got = m.layer_forward(0, torch.from_numpy(x).cuda()).cpu().numpy()
    cache = O.SequenceCache(spec, 17)
    ref = O.layer_forward(x[0].astype(np.float64), syn.FloatView(synth), spec, 0, cache, 0)
    assert_rows_close(got[0], ref, BF16_TOL, "layer output")
    k = m.cache_k(0)[0, :, :17].float().cpu().numpy()
    v = m.cache_v(0)[0, :, :17].float().cpu().numpy()
    assert_rows_close(k, cache.k[0], BF16_TOL, "K cache")
    assert_rows_close(v, cache.v[0], BF16_TOL, "V cache")


# ------------------------------------------------------------------ small bf16 stack, many tiles

@pytest.mark.parametrize("B,S", [(3, 150), (1, 1), (2, 64), (1, 50)])
def test_bf16_stack_prefill_all_positions(B, S):
    say(f"small bf16 stack prefill B={B} S={S}")
    spec = small_bf16_spec()
    m, synth = build_model(spec, 3, max_batch=4, max_seq=160, max_tokens=512)
    toks = syn.tokens(3, B, S, spec.vocab_size)
    got = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    ref, _ = O.prefill(toks, syn.FloatView(synth), spec, all_positions=True)
    assert_rows_close(got, ref, BF16_TOL, "prefill logits")
    m.sync_status()


@pytest.mark.parametrize("H,G", [(4, 4), (4, 1)])
def test_bf16_mha_and_single_kv_head(H, G):
    say(f"small bf16 stack H={H} G={G}")
    spec = small_bf16_spec(n_heads=H, n_kv_heads=G)
    m, synth = build_model(spec, 4, max_batch=2, max_seq=80, max_tokens=160)
    toks = syn.tokens(4, 2, 70, spec.vocab_size)
    got = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    ref, _ = O.prefill(toks, syn.FloatView(synth), spec, all_positions=True)
    assert_rows_close(got, ref, BF16_TOL, "prefill logits")


def test_bf16_teacher_forced_decode():
    say("small bf16 stack: prefill S=100 then 6 teacher-forced decode steps, B=3")
    spec = small_bf16_spec()
    B, S, steps = 3, 100, 6
    m, synth = build_model(spec, 5, max_batch=B, max_seq=128, max_tokens=B * S)
    toks = syn.tokens(5, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    ref0, caches = O.prefill(toks, W, spec, capacity=S + steps)
    got0 = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    assert_rows_close(got0, ref0, BF16_TOL, "prefill last logits")
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)     # teacher forcing: oracle's token
    m.sync_status()


@pytest.mark.parametrize("B", [20, 32])
def test_bf16_teacher_forced_decode_two_row_blocks(B):
    # 17..32 rows: two 16-row activation blocks (the second partly padding at B = 20), which
    # the weight-streaming GEMMs serve with more row tiles per wave (RT 2 for Q/K/V, RT 4
    # for the gate/up pair), and a split decode attention grid
    S, steps = 24, 3
    say(f"small bf16 stack: prefill S={S} then {steps} teacher-forced decode steps, B={B}")
    spec = small_bf16_spec()
    m, synth = build_model(spec, 40 + B, max_batch=B, max_seq=32, max_tokens=B * S)
    toks = syn.tokens(40 + B, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    ref0, caches = O.prefill(toks, W, spec, capacity=S + steps)
    got0 = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    assert_rows_close(got0, ref0, BF16_TOL, "prefill last logits")
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)
    m.sync_status()


def test_bf16_long_context_decode_multiple_splits():
    say("small bf16 stack: prefill S=600 (several decode splits, ragged) then 3 decode steps, B=2")
    spec = small_bf16_spec()
    B, S, steps = 2, 600, 3
    m, synth = build_model(spec, 8, max_batch=B, max_seq=640, max_tokens=B * S)
    toks = syn.tokens(8, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    ref0, caches = O.prefill(toks, W, spec, capacity=S + steps)
    got0 = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    assert_rows_close(got0, ref0, BF16_TOL, "prefill last logits")
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)


def test_bf16_generate_matches_eager_decode_steps():
    say("small bf16 stack: generate (device-side positions) vs decode steps, B=3")
    spec = small_bf16_spec()
    B, S, steps = 3, 70, 10
    m, _ = build_model(spec, 9, max_batch=B, max_seq=96, max_tokens=B * S)
    toks = torch.from_numpy(syn.tokens(9, B, S, spec.vocab_size)).cuda()
    _, first = m.prefill(toks, want_next=True)
    eager = []
    cur = first
    for k in range(steps):
        cur, _ = m.decode_step(cur, S + k, want_logits=False)
        eager.append(cur.clone())
    eager = torch.stack(eager)
    m.prefill(toks)
    out, _ = m.generate(first, S, steps)
    assert torch.equal(out, eager)
    m.prefill(toks)
    out2, lg = m.generate(first, S, steps, want_logits=True)
    assert torch.equal(out2, eager)
    assert torch.equal(lg.argmax(-1).to(torch.int32), eager)


def test_bf16_chunked_layer_forward():
    say("small bf16 layer: chunked prefill 40 + 37 + 1 tokens")
    spec = small_bf16_spec(n_layers=1)
    m, synth = build_model(spec, 6, max_batch=2, max_seq=96, max_tokens=192)
    x = syn.normal(6, "x", (2, 78, spec.dim))
    W = syn.FloatView(synth)
    outs = []
    for a, b in ((0, 40), (40, 77), (77, 78)):
        chunk = np.ascontiguousarray(x[:, a:b])
        x_in = torch.from_numpy(chunk).cuda()
        outs.append(m.layer_forward(0, x_in, start_pos=a).cpu().numpy())
        # the layer reads x_in and writes only x_out (the 2-token chunk takes the few-row
        # GEMMs, whose split-K sums are added into x_out by the FFN norm)
        np.testing.assert_array_equal(x_in.cpu().numpy(), chunk)
    got = np.concatenate(outs, axis=1)
    for bidx in range(2):
        cache = O.SequenceCache(spec, 78)
        ref = O.layer_forward(x[bidx].astype(np.float64), W, spec, 0, cache, 0)
        assert_rows_close(got[bidx], ref, BF16_TOL, f"chunked layer row {bidx}")


def test_prefill_is_deterministic():
    spec = small_bf16_spec()
    m, _ = build_model(spec, 7, max_batch=2, max_seq=128, max_tokens=256)
    toks = torch.from_numpy(syn.tokens(7, 2, 128, spec.vocab_size)).cuda()
    a = m.prefill(toks, all_positions=True)
    b = m.prefill(toks, all_positions=True)
    assert torch.equal(a, b)


def test_out_of_range_token_is_reported():
    spec = syn.TINY
    m, _ = build_model(spec, 1, max_batch=1, max_seq=16, max_tokens=16)
    bad = torch.tensor([[1, 2, spec.vocab_size + 5]], dtype=torch.int32).cuda()
    m.prefill(bad)
    with pytest.raises(bd.LlamaError) as e:
        m.sync_status()
    assert e.value.status == -1
    m.sync_status()  # cleared


# ------------------------------------------------------------------ greedy choice after prefill

@pytest.mark.parametrize("all_positions", [False, True])
def test_prefill_next_tokens_are_the_argmax_of_its_logits(all_positions):
    say(f"small bf16 stack: prefill next_tokens (all_positions={all_positions})")
    spec = small_bf16_spec()
    B, S = 3, 45
    m, synth = build_model(spec, 21, max_batch=B, max_seq=64, max_tokens=B * S)
    toks = syn.tokens(21, B, S, spec.vocab_size)
    lg, nxt = m.prefill(torch.from_numpy(toks).cuda(), all_positions=all_positions, want_next=True)
    lg = lg.cpu().numpy()
    last = lg[:, -1] if all_positions else lg
    # lowest index among equal maxima, on the GPU's own fp32 logits: bit for bit
    np.testing.assert_array_equal(nxt.cpu().numpy(), np.argmax(last, axis=-1))
    ref, _ = O.prefill(toks, syn.FloatView(synth), spec)
    check_argmax(nxt.cpu().numpy(), last, ref, "prefill next tokens")
    m.sync_status()


def test_first_call_inside_a_stream_capture_is_refused():
    # the one-time set-up (rotary table, cache fill) must run eagerly: a captured first call
    # would leave later eager calls without it
    spec = small_bf16_spec()
    m, _ = build_model(spec, 22, max_batch=2, max_seq=32, max_tokens=64)
    toks = torch.from_numpy(syn.tokens(22, 2, 1, spec.vocab_size)[:, 0].copy()).cuda()
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    st = None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            st = m.lib.llama_decode_step(m.handle, toks.data_ptr(), 2, 0, None, out.data_ptr(),
                                         bd._stream(side))
            msg = m.lib.llama_last_error().decode()
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    assert st == -1 and "capture" in msg, (st, msg)
    # eager use works afterwards and sets the model up
    nxt, lg = m.decode_step(toks, 0)
    assert np.isfinite(lg.cpu().numpy()).all()
    m.sync_status()


# ------------------------------------------------------------------ shapes off the common path

def test_bf16_ffn_width_not_a_multiple_of_128():
    # F = 1472 = 23 x 64: the down projection's K is not a multiple of 128, so at <= 32 rows
    # it takes the 128 x 32 tiled GEMM on row-major input instead of the weight-streaming one
    spec = small_bf16_spec(ffn_hidden=1472)
    B, S, steps = 4, 40, 3
    say(f"small bf16 stack F=1472: prefill {B} x {S}, {steps} teacher-forced decode steps")
    m, synth = build_model(spec, 23, max_batch=B, max_seq=48, max_tokens=B * S)
    toks = syn.tokens(23, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    ref0, caches = O.prefill(toks, W, spec, capacity=S + steps)
    got0 = m.prefill(torch.from_numpy(toks).cuda()).cpu().numpy()
    assert_rows_close(got0, ref0, BF16_TOL, "prefill logits")
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)
    m.sync_status()


def test_bf16_head_dim_64_generic_attention():
    # head_dim 64 (8 query heads over 2 KV heads at dim 512): prefill and decode attention
    # take the generic one-wave-per-row kernel in bf16
    spec = small_bf16_spec(n_heads=8, n_kv_heads=2, head_dim=64)
    B, S, steps = 2, 70, 3
    say(f"small bf16 stack d=64: prefill {B} x {S} (all positions), {steps} decode steps")
    m, synth = build_model(spec, 24, max_batch=B, max_seq=80, max_tokens=B * S)
    toks = syn.tokens(24, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    ref_all, _ = O.prefill(toks, W, spec, all_positions=True)
    got_all = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    assert_rows_close(got_all, ref_all, BF16_TOL, "prefill logits, every position")
    ref0, caches = O.prefill(toks, W, spec, capacity=S + steps)
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)
    m.sync_status()


def test_trace_records_the_residual_stream():
    # the trace holds the embedding rows bit for bit, each layer's input, and the rows the
    # final norm reads; llama_layer_forward on a recorded input reproduces the next one
    spec = small_bf16_spec()
    B, S = 2, 100
    say(f"small bf16 stack: residual-stream trace of a {B} x {S} prefill")
    m, synth = build_model(spec, 25, max_batch=B, max_seq=128, max_tokens=B * S)
    toks = syn.tokens(25, B, S, spec.vocab_size)
    tr = m.trace_hidden(B * S)
    lg = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    h = tr.cpu().numpy()
    m.trace_hidden(None)
    E = synth.as_float("tok_embeddings.weight", np.float32)
    np.testing.assert_array_equal(h[0], E[toks.reshape(-1)])
    for l in range(spec.n_layers):
        x_in = torch.from_numpy(np.ascontiguousarray(h[l].reshape(B, S, -1))).cuda()
        x_out = m.layer_forward(l, x_in).cpu().numpy().reshape(B * S, -1)
        np.testing.assert_array_equal(x_out, h[l + 1], err_msg=f"layer {l}")
    W = syn.FloatView(synth)
    assert_rows_close(lg.reshape(B * S, -1), O.head_logits(h[spec.n_layers].astype(np.float64), W, spec),
                      BF16_TOL, "head on the recorded final rows")
    m.sync_status()


def test_bf16_split_down_projection():
    # F = 8192: the down projection of a prefill of more than 64 rows, and of a decode step
    # of more than 64 sequences, is split over K in two (fp32 sums folded by the next
    # RMSNorm); the prefill against the oracle, llama_layer_forward against the recorded
    # residual stream bit for bit (it folds the sums at once), and two teacher-forced decode
    # steps at batch 80
    spec = small_bf16_spec(ffn_hidden=8192)
    B, S, DB, steps = 2, 70, 80, 2
    say(f"small bf16 stack, F=8192: prefill {B} x {S} with a residual-stream trace, then "
        f"{steps} decode steps at batch {DB}")
    m, synth = build_model(spec, 26, max_batch=DB, max_seq=S + steps, max_tokens=DB * S)
    W = syn.FloatView(synth)
    toks = syn.tokens(26, B, S, spec.vocab_size)
    tr = m.trace_hidden(B * S)
    got = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    h = tr.cpu().numpy()
    m.trace_hidden(None)
    ref, _ = O.prefill(toks, W, spec, all_positions=True)
    assert_rows_close(got, ref, BF16_TOL, "prefill logits")
    for l in range(spec.n_layers):
        x_in = torch.from_numpy(np.ascontiguousarray(h[l].reshape(B, S, -1))).cuda()
        x_out = m.layer_forward(l, x_in).cpu().numpy().reshape(B * S, -1)
        np.testing.assert_array_equal(x_out, h[l + 1], err_msg=f"layer {l}")
    dtoks = syn.tokens(27, DB, S, spec.vocab_size)
    ref0, caches = O.prefill(dtoks, W, spec, capacity=S + steps)
    got0 = m.prefill(torch.from_numpy(dtoks).cuda()).cpu().numpy()
    assert_rows_close(got0, ref0, BF16_TOL, "prefill last logits")
    cur = O.argmax(ref0).astype(np.int32)
    for k in range(steps):
        ref = O.decode_step(cur, S + k, W, spec, caches)
        nxt, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, BF16_TOL, f"decode step {k}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"decode step {k}")
        cur = O.argmax(ref).astype(np.int32)
    m.sync_status()
