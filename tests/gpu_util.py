"""Helpers shared by the GPU parity tests (not collected as tests)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from llama_decoder_forward_amd import binding as bd
from llama_decoder_forward_amd import synthetic as syn
from oracle import llama_oracle as O

BF16_TOL = 2e-2   # normwise per-row relative error, bf16 path
F32_TOL = 1e-4    # fp32 debug path


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    bd.load_library()  # raises if the HIP library is missing: no fallback


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def build_model(spec, seed, max_batch, max_seq, max_tokens, cache=True):
    synth = syn.SyntheticWeights(spec, seed, cache=cache)
    w = bd.upload_weights(synth)
    m = bd.Model(spec, w, max_batch=max_batch, max_seq=max_seq, max_tokens=max_tokens)
    return m, synth


def rowwise_rel(gpu, ref):
    """max_i |g_i - o_i| / max_i |o_i| for each row (last axis)."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    o = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    return np.max(np.abs(g - o), axis=1) / np.maximum(np.max(np.abs(o), axis=1), 1e-30)


def assert_rows_close(gpu, ref, tol, what=""):
    r = rowwise_rel(gpu, ref)
    worst = int(np.argmax(r))
    assert np.all(np.isfinite(np.asarray(gpu))), f"{what}: non-finite GPU values"
    assert r.max() <= tol, f"{what}: row {worst} normwise rel err {r.max():.3e} > {tol}"
    return r


def check_argmax(gpu_tokens, gpu_logits, ref_logits, what=""):
    """GPU argmax equals argmax of the GPU's own logits (strict); against the oracle a
    difference is allowed only where the oracle's top-2 margin is within twice the row's
    measured error (a near tie)."""
    gl = np.asarray(gpu_logits, dtype=np.float64)
    rl = np.asarray(ref_logits, dtype=np.float64)
    gt = np.asarray(gpu_tokens).reshape(-1)
    gl2 = gl.reshape(-1, gl.shape[-1])
    rl2 = rl.reshape(-1, rl.shape[-1])
    np.testing.assert_array_equal(gt, np.argmax(gl2, axis=-1), err_msg=f"{what}: argmax of own logits")
    ref_tok = np.argmax(rl2, axis=-1)
    flips = 0
    for i in range(len(gt)):
        if gt[i] != ref_tok[i]:
            e = np.max(np.abs(gl2[i] - rl2[i]))
            top = np.sort(rl2[i])[-2:]
            margin = top[1] - top[0]
            assert margin <= 2 * e, f"{what}: row {i} argmax {gt[i]} != {ref_tok[i]} with margin {margin:.3e} > 2*err {2*e:.3e}"
            flips += 1
    return flips


def small_bf16_spec(**over):
    base = syn.ModelSpec(dim=512, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=128,
                         ffn_hidden=1536, vocab_size=1024, dtype="bf16")
    return dataclasses.replace(base, **over)
