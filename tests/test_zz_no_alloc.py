"""llama_decode_step_noalloc (scratch in the library's static array) against
llama_decode_step (scratch in the model's workspace), through the C ABI: the same tokens and
logits bit for bit, on two calls in a row, the second with a smaller batch."""
import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import synthetic as syn

from gpu_util import build_model, require_gpu, say, small_bf16_spec

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(m, toks, pos, want_logits):
    """(tokens, logits) of llama_decode_step and of llama_decode_step_noalloc for the same
    step.  Each call writes the same key and value at pos before it attends."""
    n1, l1 = m.decode_step(toks, pos, want_logits=want_logits)
    n2, l2 = m.decode_step_noalloc(toks, pos, want_logits=want_logits)
    torch.cuda.synchronize()
    return n1, l1, n2, l2


@pytest.mark.parametrize("spec_name,B1,B2,ctx", [
    # small stack: split-K residual sums, split decode attention with partials and merge
    ("small", 8, 3, 300),
    # 8B widths, one layer: batch 32 takes whole-context attention workgroups, batch 4 the
    # split path over 4096 keys
    ("8b_layer", 32, 4, 4096),
])
def test_noalloc_matches_workspace_decode(spec_name, B1, B2, ctx):
    spec = small_bf16_spec() if spec_name == "small" else syn.LLAMA3_8B_ONE_LAYER
    say(f"noalloc vs workspace decode: {spec_name}, batch {B1} then {B2}, context {ctx}")
    m, _ = build_model(spec, 27, max_batch=B1, max_seq=ctx + 2, max_tokens=B1 * ctx,
                       cache=(spec_name == "small"))
    toks = syn.tokens(27, B1, ctx + 2, spec.vocab_size)
    _, first = m.prefill(torch.from_numpy(np.ascontiguousarray(toks[:, :ctx])).cuda(),
                         want_next=True)
    # first call: the whole batch, with logits
    n1, l1, n2, l2 = _pair(m, first, ctx, True)
    assert torch.equal(n1, n2), "next tokens differ"
    assert torch.equal(l1, l2), "logits differ"
    # the same step without logits (the step's logits then live in the scratch array too)
    n3, _, n4, _ = _pair(m, first, ctx, False)
    assert torch.equal(n3, n1) and torch.equal(n4, n1)
    # second call: a smaller batch at the next position
    cur = n1[:B2].contiguous()
    n1, l1, n2, l2 = _pair(m, cur, ctx + 1, True)
    assert torch.equal(n1, n2), "next tokens differ (smaller batch)"
    assert torch.equal(l1, l2), "logits differ (smaller batch)"
    np.testing.assert_array_equal(n2.cpu().numpy(), np.argmax(l2.cpu().numpy(), axis=-1))
    m.sync_status()


def test_noalloc_refuses_a_step_beyond_its_scratch():
    # 64 sequences of 4 heads over up to 131072 positions: 513 split partials of 130 floats
    # per (sequence, head), 68 MB, more than the 64 MiB array holds
    spec = small_bf16_spec(n_layers=1)
    m, _ = build_model(spec, 28, max_batch=64, max_seq=131072, max_tokens=64)
    toks = torch.zeros(64, dtype=torch.int32, device="cuda")
    m.decode_step(toks[:1].contiguous(), 0)       # set-up on the workspace path
    from llama_decoder_forward_amd import binding as bd
    with pytest.raises(bd.LlamaError) as e:
        m.decode_step_noalloc(toks, 10)
    assert e.value.status == -3 and "scratch" in str(e.value)
    m.sync_status()
