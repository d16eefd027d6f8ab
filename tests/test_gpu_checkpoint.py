"""A model whose weights come through the checkpoint front end (consolidated.00.pth and
params.json, the layout the article loads in section 下载并读取模型权重) runs the same
bytes as one built from the weights directly, and matches the oracle."""
import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import binding as bd
from llama_decoder_forward_amd import checkpoint as ck
from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

from gpu_util import BF16_TOL, assert_rows_close, build_model, require_gpu, say, small_bf16_spec

# a hung GPU call ends the run (thread method) instead of stalling it
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300, method="thread")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_checkpoint_loaded_model_matches_direct_weights_and_oracle(tmp_path):
    spec = small_bf16_spec()  # dim 512, FFN 1536 = multiple_of 512 over 2*4*512/3
    say("small bf16 stack written as consolidated.00.pth + params.json, loaded, prefill 2 x 40")
    synth = syn.SyntheticWeights(spec, 12)
    tensors = {n: torch.from_numpy(synth.stored(n).view(np.int16).copy()).view(torch.bfloat16)
               for n in synth.names()}
    ck.save_checkpoint(str(tmp_path), spec, tensors, multiple_of=512)
    spec2, w = ck.load_checkpoint(str(tmp_path), device="cuda")
    assert spec2 == spec
    toks = torch.from_numpy(syn.tokens(12, 2, 40, spec.vocab_size)).cuda()
    m = bd.Model(spec2, w, max_batch=2, max_seq=64, max_tokens=128)
    got = m.prefill(toks, all_positions=True).cpu().numpy()
    m.sync_status()
    m.free()
    m2, _ = build_model(spec, 12, max_batch=2, max_seq=64, max_tokens=128)
    direct = m2.prefill(toks, all_positions=True).cpu().numpy()
    m2.free()
    np.testing.assert_array_equal(got, direct)
    ref, _ = O.prefill(toks.cpu().numpy(), syn.FloatView(synth), spec, all_positions=True)
    assert_rows_close(got, ref, BF16_TOL, "checkpoint-loaded prefill logits")
