"""GPU parity of chunked prefill (llama_prefill_at) and ragged decode
(llama_decode_step_ragged) against the CPU oracle, through the C ABI.

Chunked prefill continues every sequence at start_pos into the cache the earlier chunks
wrote; ragged decode gives every sequence its own position (device memory).  The oracle side
is its per-sequence calls: prefill_sequence_at for a chunk, decode_sequence_step with that
row's position.
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


def _chunks_vs_oracle(spec, seed, B, bounds, tol, max_seq):
    m, synth = build_model(spec, seed, max_batch=B, max_seq=max_seq, max_tokens=B * max_seq)
    S = bounds[-1][1]
    toks = syn.tokens(seed, B, S, spec.vocab_size)
    ref, _ = O.prefill(toks, syn.FloatView(synth), spec, all_positions=True,
                       dtype=np.float64 if tol == F32_TOL else np.float32)
    for a, b in bounds:
        chunk = torch.from_numpy(np.ascontiguousarray(toks[:, a:b])).cuda()
        got = m.prefill(chunk, all_positions=True, start_pos=a).cpu().numpy()
        assert_rows_close(got.reshape(-1, spec.vocab_size), ref[:, a:b].reshape(-1, spec.vocab_size),
                          tol, f"chunk [{a},{b})")
        # last-position mode of the same chunk (rewrites the same cache entries); in bf16 its
        # vocabulary GEMM has B rows, not B*S, and may sum in another order
        last = m.prefill(chunk, start_pos=a).cpu().numpy()
        if tol == F32_TOL:
            np.testing.assert_array_equal(last, got[:, -1])
        assert_rows_close(last, ref[:, b - 1], tol, f"chunk [{a},{b}) last position")
    m.sync_status()


def test_tiny_fp32_prefill_at_chunks():
    say("tiny fp32: prefill of 17 tokens as chunks [0,6) [6,11) [11,17), B=2")
    _chunks_vs_oracle(syn.TINY, 11, 2, ((0, 6), (6, 11), (11, 17)), F32_TOL, 32)


def test_bf16_prefill_at_chunks():
    # 70-token chunks take the tiled GEMMs and flash attention with start_pos > 0; the last
    # one-token chunk takes the few-row GEMMs.
    say("small bf16 stack: prefill of 131 tokens as chunks 70 + 60 + 1, B=2")
    _chunks_vs_oracle(small_bf16_spec(), 12, 2, ((0, 70), (70, 130), (130, 131)), BF16_TOL, 160)


def test_bf16_prefill_at_chunks_inside_a_key_block():
    # four query heads per KV head (32 positions per query tile) and chunks that start
    # inside a 64-key block: a chunk's first query tile then meets a key block whose keys
    # all lie past the positions of some of its rows, with no earlier key seen by those
    # rows in the same pass (the case the exponentials must take against 0, not -inf)
    say("bf16 stack, 8 query heads / 2 KV heads: prefill of 130 tokens as chunks 40 + 32 + 58, B=2")
    spec = small_bf16_spec(dim=1024, n_heads=8, n_kv_heads=2)
    _chunks_vs_oracle(spec, 13, 2, ((0, 40), (40, 72), (72, 130)), BF16_TOL, 160)


@pytest.mark.parametrize("H,G", [(16, 2), (16, 1)])
def test_bf16_prefill_at_chunks_wide_groups(H, G):
    # 8 and 16 query heads per KV head (16 and 8 positions per 128-row query tile), from
    # position 0 and from a start inside a key block
    say(f"bf16 stack, {H} query heads / {G} KV heads: prefill of 150 tokens as chunks 37 + 113, B=2")
    spec = small_bf16_spec(dim=128 * H, n_heads=H, n_kv_heads=G)
    _chunks_vs_oracle(spec, 14, 2, ((0, 37), (37, 150)), BF16_TOL, 160)


def _ragged_vs_oracle(spec, seed, B, S, positions, steps, tol, max_seq):
    m, synth = build_model(spec, seed, max_batch=B, max_seq=max_seq, max_tokens=B * S)
    toks = syn.tokens(seed, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    dt = np.float64 if tol == F32_TOL else np.float32
    m.prefill(torch.from_numpy(toks).cuda())
    # oracle caches of each row's prefix 0..pos-1; entries past a row's position, which the
    # GPU cache still holds from the longer prefill, must be ignored
    caches = []
    for b, p in enumerate(positions):
        c = O.SequenceCache(spec, max_seq, dt)
        if p > 0:
            O.prefill_sequence_at(toks[b, :p], 0, W, spec, c, dtype=dt)
        caches.append(c)
    pos = np.array(positions, dtype=np.int32)
    cur = np.array([toks[b, p] for b, p in enumerate(positions)], dtype=np.int32)
    for k in range(steps):
        ref = np.stack([O.decode_sequence_step(int(cur[b]), int(pos[b]), W, spec, caches[b], dt)
                        for b in range(B)])
        nxt, lg = m.decode_step_ragged(torch.from_numpy(cur).cuda(), torch.from_numpy(pos).cuda())
        lg = lg.cpu().numpy()
        assert_rows_close(lg, ref, tol, f"ragged step {k} at {pos.tolist()}")
        check_argmax(nxt.cpu().numpy(), lg, ref, f"ragged step {k}")
        cur = O.argmax(ref).astype(np.int32)   # teacher forcing
        pos = pos + 1
    m.sync_status()


def test_tiny_fp32_ragged_decode():
    say("tiny fp32: ragged decode at positions 4, 12, 9, 0 after a 13-token prefill, 3 steps")
    _ragged_vs_oracle(syn.TINY, 13, 4, 13, (4, 12, 9, 0), 3, F32_TOL, 24)


def test_bf16_ragged_decode():
    say("small bf16 stack: ragged decode at positions 37, 99, 300, 1, 3 steps, B=4")
    _ragged_vs_oracle(small_bf16_spec(), 14, 4, 310, (37, 99, 300, 1), 3, BF16_TOL, 320)


def test_ragged_position_out_of_range_is_reported():
    # A device position outside [0, max_seq) raises the call's flag; the other rows still
    # decode correctly and that row's cache is left as it was.
    say("tiny fp32: ragged decode with one position past max_seq")
    spec = syn.TINY
    B, S, max_seq = 2, 9, 16
    m, synth = build_model(spec, 15, max_batch=B, max_seq=max_seq, max_tokens=B * S)
    toks = syn.tokens(15, B, S, spec.vocab_size)
    m.prefill(torch.from_numpy(toks).cuda())
    k_before = m.cache_k(0)[1].clone()
    W = syn.FloatView(synth)
    c0 = O.SequenceCache(spec, max_seq)
    O.prefill_sequence_at(toks[0, :5], 0, W, spec, c0)
    ref0 = O.decode_sequence_step(int(toks[0, 5]), 5, W, spec, c0)
    cur = torch.tensor([toks[0, 5], 3], dtype=torch.int32).cuda()
    pos = torch.tensor([5, max_seq + 7], dtype=torch.int32).cuda()
    _, lg = m.decode_step_ragged(cur, pos)
    with pytest.raises(bd.LlamaError) as e:
        m.sync_status()
    assert e.value.status == -1 and "position" in str(e.value)
    assert_rows_close(lg.cpu().numpy()[:1], ref0[None], F32_TOL, "valid row")
    assert torch.equal(m.cache_k(0)[1], k_before)
    m.sync_status()  # cleared
