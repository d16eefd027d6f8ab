"""GPU parity at model widths past the 8B shape's 4096, through the C ABI.

The RMSNorm kernel picks its block by width: one 8-value chunk per thread of 256, 512 or
1024 threads up to dim 8192, two chunks per thread of 1024 above that.  The decode
residual GEMMs' split count falls with the width (3 splits at dim 6144, 2 at 12288), so
the folding RMSNorm also takes split counts that are not a multiple of four.  One layer,
small FFN and vocabulary, prefill of all positions, then teacher-forced decode steps, each
compared with the oracle (float64 on the same bf16 weights) within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

from gpu_util import BF16_TOL, assert_rows_close, build_model, require_gpu, say, small_bf16_spec

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# (dim, query heads, KV heads): head_dim 128, query group of 4 (the MFMA attention path)
@pytest.mark.parametrize("D,H,G", [(6144, 48, 12), (12288, 96, 24)])
def test_wide_dim_prefill_and_decode(D, H, G):
    B, S, steps = 2, 9, 2
    say(f"bf16 one layer dim {D}, H={H}, G={G}: prefill B={B} S={S}, {steps} decode steps")
    spec = small_bf16_spec(dim=D, n_heads=H, n_kv_heads=G, n_layers=1, ffn_hidden=1024,
                           vocab_size=512)
    m, synth = build_model(spec, 21, max_batch=B, max_seq=32, max_tokens=B * S, cache=False)
    toks = syn.tokens(21, B, S, spec.vocab_size)
    W = syn.FloatView(synth)
    got = m.prefill(torch.from_numpy(toks).cuda(), all_positions=True).cpu().numpy()
    ref, _ = O.prefill(toks, W, spec, all_positions=True)
    assert_rows_close(got.reshape(B * S, -1), ref.reshape(B * S, -1), BF16_TOL, "prefill logits")
    _, caches = O.prefill(toks, W, spec, capacity=S + steps)
    cur = np.argmax(ref[:, -1], axis=-1).astype(np.int32)
    for k in range(steps):
        say(f"  decode step {k}")
        want = O.decode_step(cur, S + k, W, spec, caches)
        _, lg = m.decode_step(torch.from_numpy(cur).cuda(), S + k)
        assert_rows_close(lg.cpu().numpy(), want, BF16_TOL, f"decode step {k}")
        cur = np.argmax(want, axis=-1).astype(np.int32)
    m.sync_status()
    m.free()
