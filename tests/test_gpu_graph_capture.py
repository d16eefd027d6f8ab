"""Decode calls recorded into a HIP stream capture and replayed, through the C ABI.

After a model's first call (which does its one-time set-up), llama_generate and
llama_decode_step_ragged enqueue kernel launches only: no memset, no allocation, no host
synchronisation.  A serving loop can therefore capture them into a graph and replay it.
Each replay here runs after eager work on the same model and must reproduce the eager
call's tokens and logits bit for bit.
"""
import pytest
import torch

from llama_decoder_forward_amd import binding as bd
from llama_decoder_forward_amd import synthetic as syn

from gpu_util import build_model, require_gpu, say, small_bf16_spec

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def test_generate_replays_from_a_graph():
    B, S, N = 3, 40, 5
    say(f"small bf16 stack: generate {N} steps at B={B} captured in a HIP graph")
    spec = small_bf16_spec()
    m, _ = build_model(spec, 31, max_batch=B, max_seq=64, max_tokens=B * S)
    toks = torch.from_numpy(syn.tokens(31, B, S, spec.vocab_size)).cuda()
    _, first = m.prefill(toks, want_next=True)
    out = torch.empty((N, B), dtype=torch.int32, device="cuda")
    lg = torch.empty((N, B, spec.vocab_size), dtype=torch.float32, device="cuda")

    def eager(stream=None):
        bd.check(m.lib.llama_generate(m.handle, first.data_ptr(), B, S, N, out.data_ptr(),
                                      lg.data_ptr(), bd._stream(stream)))

    eager()
    torch.cuda.synchronize()
    ref_tok, ref_lg = out.clone(), lg.clone()
    g = _capture(eager)
    for r in range(3):
        out.zero_()
        lg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_tok), f"replay {r}: tokens differ"
        assert torch.equal(lg, ref_lg), f"replay {r}: logits differ"
        # eager work on the same model between replays
        m.decode_step(first, S)
        torch.cuda.synchronize()
    m.sync_status()
    m.free()


def test_ragged_decode_replays_from_a_graph():
    B, S = 4, 48
    say(f"small bf16 stack: ragged decode step at B={B} captured in a HIP graph")
    spec = small_bf16_spec()
    m, _ = build_model(spec, 32, max_batch=B, max_seq=64, max_tokens=B * S)
    toks = torch.from_numpy(syn.tokens(32, B, S, spec.vocab_size)).cuda()
    m.prefill(toks)
    cur = torch.from_numpy(syn.tokens(33, B, 1, spec.vocab_size)[:, 0].copy()).cuda()
    pos = torch.tensor([S - 9, S - 1, S - 30, S - 4], dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, spec.vocab_size), dtype=torch.float32, device="cuda")

    def step(stream=None):
        m.decode_step_ragged(cur, pos, next_tokens=nxt, logits=lg, stream=stream)

    step()
    torch.cuda.synchronize()
    ref_tok, ref_lg = nxt.clone(), lg.clone()
    g = _capture(step)
    for r in range(3):
        nxt.zero_()
        lg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(nxt, ref_tok), f"replay {r}: tokens differ"
        assert torch.equal(lg, ref_lg), f"replay {r}: logits differ"
        step()
        torch.cuda.synchronize()
    m.sync_status()
    m.free()


def test_decode_step_replays_from_a_graph():
    B, S = 2, 33
    say(f"small bf16 stack: decode step at B={B}, position {S}, captured in a HIP graph")
    spec = small_bf16_spec()
    m, _ = build_model(spec, 34, max_batch=B, max_seq=64, max_tokens=B * S)
    toks = torch.from_numpy(syn.tokens(34, B, S, spec.vocab_size)).cuda()
    _, cur = m.prefill(toks, want_next=True)
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, spec.vocab_size), dtype=torch.float32, device="cuda")

    def step(stream=None):
        m.decode_step(cur, S, next_tokens=nxt, logits=lg, stream=stream)

    step()
    torch.cuda.synchronize()
    ref_tok, ref_lg = nxt.clone(), lg.clone()
    g = _capture(step)
    for r in range(3):
        nxt.zero_()
        lg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(nxt, ref_tok), f"replay {r}: tokens differ"
        assert torch.equal(lg, ref_lg), f"replay {r}: logits differ"
        step()
        torch.cuda.synchronize()
    m.sync_status()
    m.free()
