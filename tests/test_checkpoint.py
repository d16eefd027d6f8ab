"""The checkpoint front end (no GPU): params.json to model shape, and a state dict in the
layout the article loads (section 下载并读取模型权重 of "250 lines of code to build Llama 3
from scratch") read back bit-exactly, with every malformed case refused."""
import dataclasses
import json
import os
import pickle

import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import checkpoint as ck
from llama_decoder_forward_amd import synthetic as syn


def test_params_printed_in_the_article_give_the_8b_shape():
    # the params.json the article prints for Meta-Llama-3-8B, with the 14336 rows of W1
    params = {"dim": 4096, "n_layers": 32, "n_heads": 32, "n_kv_heads": 8, "vocab_size": 128256,
              "multiple_of": 1024, "ffn_dim_multiplier": 1.3, "norm_eps": 1e-05,
              "rope_theta": 500000.0}
    spec = ck.spec_from_params(params, 14336)
    assert spec == syn.LLAMA3_8B


def test_stored_ffn_width_must_agree_with_params():
    params = {"dim": 4096, "n_layers": 1, "n_heads": 32, "n_kv_heads": 8, "vocab_size": 128256,
              "multiple_of": 1024, "ffn_dim_multiplier": 1.3}
    assert ck.spec_from_params(params, 14336).ffn_hidden == 14336
    # not a multiple of 1024; one block short of 14198 (rounded down); one block too many;
    # the width without the multiplier
    for bad in (14335, 13312, 15360, 11264, 0):
        with pytest.raises(ck.CheckpointError):
            ck.spec_from_params(params, bad)
    # the same rule agrees with the oracle's FFN-width helper over many shapes
    from oracle import llama_oracle as O
    for dim in (64, 128, 512, 1000, 4096, 5120, 8192):
        for mo in (32, 64, 256, 1024):
            for mult in (None, 1.0, 1.3, 1.5):
                w = O.ffn_hidden_size(dim, mo, mult)
                p = {"dim": dim, "multiple_of": mo, "ffn_dim_multiplier": mult}
                assert ck.params_admit_ffn_width(p, w)
                assert not ck.params_admit_ffn_width(p, w + mo)
                assert not ck.params_admit_ffn_width(p, w - mo)
    # without multiple_of the stored width is taken as is
    p2 = {k: v for k, v in params.items() if k != "multiple_of"}
    assert ck.spec_from_params(p2, 1000).ffn_hidden == 1000


def _tensors(synth):
    out = {}
    for name in synth.names():
        a = synth.stored(name)
        if synth.spec.dtype == "bf16":
            out[name] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(a.copy())
    return out


SMALL = syn.ModelSpec(dim=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=32, ffn_hidden=384,
                      vocab_size=96, dtype="bf16")  # multiple_of 128: 2*4*128/3 = 341 -> 384


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_round_trip_is_bit_exact(tmp_path, dtype):
    synth = syn.SyntheticWeights(SMALL, 7)
    tensors = _tensors(synth)
    ck.save_checkpoint(str(tmp_path), SMALL, tensors, multiple_of=128)
    spec, w = ck.load_checkpoint(str(tmp_path), dtype=dtype, device="cpu")
    assert spec == dataclasses.replace(SMALL, dtype=dtype)
    assert set(w) == set(tensors)
    for name, t in tensors.items():
        got = w[name]
        assert got.dtype == (torch.bfloat16 if dtype == "bf16" else torch.float32)
        # bf16 -> f32 widening is exact, so both must equal the stored values
        np.testing.assert_array_equal(got.float().numpy(), t.float().numpy())


def test_safetensors_file_is_read(tmp_path):
    from safetensors.torch import save_file
    synth = syn.SyntheticWeights(SMALL, 8)
    tensors = _tensors(synth)
    save_file(tensors, str(tmp_path / "model.safetensors"))
    with open(tmp_path / "params.json", "w") as f:
        json.dump({"dim": 128, "n_layers": 2, "n_heads": 4, "n_kv_heads": 2, "vocab_size": 96,
                   "multiple_of": 128}, f)
    spec, w = ck.load_checkpoint(str(tmp_path), device="cpu")
    assert spec == SMALL
    np.testing.assert_array_equal(w["output.weight"].float().numpy(),
                                  tensors["output.weight"].float().numpy())


def _write(tmp_path, tensors, params=None):
    torch.save(tensors, str(tmp_path / "consolidated.00.pth"))
    with open(tmp_path / "params.json", "w") as f:
        json.dump(params or {"dim": 128, "n_layers": 2, "n_heads": 4, "n_kv_heads": 2,
                             "vocab_size": 96, "multiple_of": 128}, f)


def test_missing_extra_and_misshapen_tensors_are_refused(tmp_path):
    tensors = _tensors(syn.SyntheticWeights(SMALL, 9))
    t = dict(tensors)
    del t["layers.1.ffn_norm.weight"]
    _write(tmp_path, t)
    with pytest.raises(ck.CheckpointError, match="missing"):
        ck.load_checkpoint(str(tmp_path), device="cpu")
    t = dict(tensors)
    t["layers.2.ffn_norm.weight"] = t["layers.1.ffn_norm.weight"]
    _write(tmp_path, t)
    with pytest.raises(ck.CheckpointError, match="unexpected"):
        ck.load_checkpoint(str(tmp_path), device="cpu")
    t = dict(tensors)
    t["layers.1.attention.wk.weight"] = t["layers.1.attention.wq.weight"]  # [128,128], not [64,128]
    _write(tmp_path, t)
    with pytest.raises(ck.CheckpointError, match="shape"):
        ck.load_checkpoint(str(tmp_path), device="cpu")
    t = dict(tensors)
    t["norm.weight"] = torch.ones(128, dtype=torch.int32)
    _write(tmp_path, t)
    with pytest.raises(ck.CheckpointError, match="floating"):
        ck.load_checkpoint(str(tmp_path), device="cpu")


def test_missing_params_and_sharded_checkpoints_are_refused(tmp_path):
    tensors = _tensors(syn.SyntheticWeights(SMALL, 10))
    torch.save(tensors, str(tmp_path / "consolidated.00.pth"))
    with pytest.raises(ck.CheckpointError, match="params.json"):
        ck.load_checkpoint(str(tmp_path), device="cpu")
    _write(tmp_path, tensors)
    torch.save(tensors, str(tmp_path / "consolidated.01.pth"))
    with pytest.raises(ck.CheckpointError, match="shards"):
        ck.load_checkpoint(str(tmp_path), device="cpu")


class _NotATensor:
    """A pickled object: loading it would need code from the file."""


def test_pickled_objects_are_not_loaded(tmp_path):
    tensors = _tensors(syn.SyntheticWeights(SMALL, 11))
    tensors["norm.weight"] = _NotATensor()
    torch.save(tensors, str(tmp_path / "consolidated.00.pth"))
    with open(tmp_path / "params.json", "w") as f:
        json.dump({"dim": 128, "n_layers": 2, "n_heads": 4, "n_kv_heads": 2, "vocab_size": 96,
                   "multiple_of": 128}, f)
    with pytest.raises(pickle.UnpicklingError):
        ck.load_checkpoint(str(tmp_path), device="cpu")
