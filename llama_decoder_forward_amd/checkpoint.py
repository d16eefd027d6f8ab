"""Loading weights stored the way the article reads them.

The article "250 lines of code to build Llama 3 from scratch" (ai02.cc), section
下载并读取模型权重 (loading the weights), reads Meta's checkpoint directory:

* ``consolidated.00.pth``, a state dict keyed ``tok_embeddings.weight``,
  ``layers.{i}.attention.{wq,wk,wv,wo}.weight``, ``layers.{i}.feed_forward.{w1,w3,w2}.weight``,
  ``layers.{i}.attention_norm.weight``, ``layers.{i}.ffn_norm.weight``, ``norm.weight`` and
  ``output.weight``; matrices are [out, in];
* ``params.json`` with dim, n_layers, n_heads, n_kv_heads, vocab_size, multiple_of,
  ffn_dim_multiplier, norm_eps and rope_theta.

:func:`load_checkpoint` reads such a directory (or the same keys in one ``.safetensors``
file next to ``params.json``). It checks that every tensor is present and has the shape
params.json implies. It converts each to the storage type (bf16, or fp32 for the debug
precision) and returns the ``{name: device tensor}`` dict that :class:`binding.Model`
takes.

``.pth`` files are read with ``torch.load(weights_only=True)``, which executes nothing
from the file, and memory-mapped, so the host holds one tensor at a time. Nothing here
computes the model. :func:`save_checkpoint` writes the same layout (used to make test
checkpoints from synthetic weights).
"""
from __future__ import annotations

import glob
import json
import os

import torch

from .synthetic import ModelSpec

class CheckpointError(ValueError):
    """A checkpoint directory that does not hold the expected tensors."""


def params_admit_ffn_width(params: dict, width: int) -> bool:
    """Whether a stored SwiGLU width agrees with params.json.

    params.json names no width, only ``multiple_of`` and ``ffn_dim_multiplier``.  The
    stored width must be a whole number of ``multiple_of`` blocks, and the smallest such
    number that still covers the SwiGLU width of the recipe: two thirds of four times
    dim, scaled by the multiplier (so that width - multiple_of falls short of it).  With no
    ``multiple_of`` in the file nothing is checked.
    """
    if "multiple_of" not in params:
        return True
    block = int(params["multiple_of"])
    need = (8 * int(params["dim"])) // 3
    if params.get("ffn_dim_multiplier") is not None:
        need = int(float(params["ffn_dim_multiplier"]) * need)
    return block > 0 and width % block == 0 and width - block < need <= width


def spec_from_params(params: dict, ffn_hidden: int, dtype: str = "bf16") -> ModelSpec:
    """ModelSpec of a params.json dict and the stored SwiGLU width (the rows of
    ``layers.0.feed_forward.w1.weight``), which must agree with params.json."""
    try:
        dim, n_layers, n_heads = int(params["dim"]), int(params["n_layers"]), int(params["n_heads"])
        vocab = int(params["vocab_size"])
    except KeyError as e:
        raise CheckpointError(f"params.json lacks {e.args[0]!r}") from None
    n_kv = int(params.get("n_kv_heads") or n_heads)
    if dim <= 0 or n_heads <= 0 or dim % n_heads != 0 or n_heads % n_kv != 0 or vocab <= 0:
        raise CheckpointError(f"inconsistent params: dim {dim}, n_heads {n_heads}, "
                              f"n_kv_heads {n_kv}, vocab_size {vocab}")
    if ffn_hidden <= 0 or not params_admit_ffn_width(params, ffn_hidden):
        raise CheckpointError(f"stored FFN width {ffn_hidden} does not follow from params.json "
                              f"(multiple_of {params.get('multiple_of')}, ffn_dim_multiplier "
                              f"{params.get('ffn_dim_multiplier')})")
    return ModelSpec(dim=dim, n_layers=n_layers, n_heads=n_heads, n_kv_heads=n_kv,
                     head_dim=dim // n_heads, ffn_hidden=int(ffn_hidden), vocab_size=vocab,
                     norm_eps=float(params.get("norm_eps", 1e-5)),
                     rope_theta=float(params.get("rope_theta", 500000.0)), dtype=dtype)


def expected_shapes(spec: ModelSpec) -> dict:
    """Tensor name -> shape ([out, in] matrices) of a checkpoint of this spec."""
    D, d, H, G, F, V = spec.dim, spec.head_dim, spec.n_heads, spec.n_kv_heads, spec.ffn_hidden, spec.vocab_size
    shapes = {"tok_embeddings.weight": (V, D), "norm.weight": (D,), "output.weight": (V, D)}
    per_layer = {"attention.wq.weight": (H * d, D), "attention.wk.weight": (G * d, D),
                 "attention.wv.weight": (G * d, D), "attention.wo.weight": (D, H * d),
                 "feed_forward.w1.weight": (F, D), "feed_forward.w3.weight": (F, D),
                 "feed_forward.w2.weight": (D, F), "attention_norm.weight": (D,),
                 "ffn_norm.weight": (D,)}
    for l in range(spec.n_layers):
        for k, s in per_layer.items():
            shapes[f"layers.{l}.{k}"] = s
    return shapes


def _open_state(directory: str):
    """(state dict of tensors, source file) of the single weights file of a directory."""
    pths = sorted(glob.glob(os.path.join(directory, "consolidated.*.pth")))
    sts = sorted(glob.glob(os.path.join(directory, "*.safetensors")))
    if len(pths) > 1:
        raise CheckpointError(f"{len(pths)} consolidated.*.pth shards: model-parallel shards "
                              "are not merged here; give a single-file checkpoint")
    if pths:
        return torch.load(pths[0], map_location="cpu", weights_only=True, mmap=True), pths[0]
    if len(sts) == 1:
        from safetensors.torch import load_file
        return load_file(sts[0], device="cpu"), sts[0]
    raise CheckpointError(f"no consolidated.00.pth (or single .safetensors) in {directory}")


def load_checkpoint(directory: str, dtype: str = "bf16", device="cuda"):
    """(ModelSpec, {name: tensor on device}) of the checkpoint in ``directory``.

    dtype is the storage type of the weights handed to the library: "bf16" (the
    checkpoint's own type) or "f32" (the debug precision). Raises CheckpointError for a
    missing params.json, a missing or misshapen tensor, or an unexpected key."""
    if dtype not in ("bf16", "f32"):
        raise CheckpointError(f"dtype {dtype!r}: use 'bf16' or 'f32'")
    ppath = os.path.join(directory, "params.json")
    if not os.path.isfile(ppath):
        raise CheckpointError(f"no params.json in {directory}")
    with open(ppath) as f:
        params = json.load(f)
    state, src = _open_state(directory)
    w1 = state.get("layers.0.feed_forward.w1.weight")
    if w1 is None or w1.dim() != 2:
        raise CheckpointError(f"{src}: missing or misshapen layers.0.feed_forward.w1.weight")
    spec = spec_from_params(params, int(w1.shape[0]), dtype)
    shapes = expected_shapes(spec)
    missing = [k for k in shapes if k not in state]
    extra = [k for k in state if k not in shapes]
    if missing or extra:
        raise CheckpointError(f"{src}: missing {missing[:5]}{'...' if len(missing) > 5 else ''}, "
                              f"unexpected {extra[:5]}{'...' if len(extra) > 5 else ''}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name, shape in shapes.items():
        t = state[name]
        if tuple(t.shape) != shape:
            raise CheckpointError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
        if not t.is_floating_point():
            raise CheckpointError(f"{name}: dtype {t.dtype} is not floating point")
        out[name] = t.to(dtype=tdt).contiguous().to(device)
    return spec, out


def save_checkpoint(directory: str, spec: ModelSpec, tensors: dict, multiple_of: int | None = None,
                    ffn_dim_multiplier=None) -> None:
    """Write ``tensors`` ({name: torch tensor}, the keys of expected_shapes(spec)) as
    consolidated.00.pth plus params.json. multiple_of / ffn_dim_multiplier are recorded
    when given and must reproduce spec.ffn_hidden."""
    shapes = expected_shapes(spec)
    if set(tensors) != set(shapes):
        raise CheckpointError("tensors do not match the spec's keys")
    params = {"dim": spec.dim, "n_layers": spec.n_layers, "n_heads": spec.n_heads,
              "n_kv_heads": spec.n_kv_heads, "vocab_size": spec.vocab_size,
              "norm_eps": spec.norm_eps, "rope_theta": spec.rope_theta}
    if multiple_of is not None:
        params["multiple_of"] = multiple_of
        params["ffn_dim_multiplier"] = ffn_dim_multiplier
        if not params_admit_ffn_width(params, spec.ffn_hidden):
            raise CheckpointError("multiple_of / ffn_dim_multiplier do not admit spec.ffn_hidden")
    os.makedirs(directory, exist_ok=True)
    torch.save({k: tensors[k] for k in shapes}, os.path.join(directory, "consolidated.00.pth"))
    with open(os.path.join(directory, "params.json"), "w") as f:
        json.dump(params, f)
