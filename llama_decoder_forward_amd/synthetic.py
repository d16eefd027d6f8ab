"""Seeded synthetic inputs for the Llama-3 decoder forward pass.

This module is neutral data preparation shared by the GPU path's tests and benchmark
and by the CPU oracle's tests.  It holds none of the model's arithmetic: it only draws
random numbers, rounds them to the storage type and names the tensors.

Recipe (the same for every caller):

* Every tensor is drawn from numpy's PCG64, seeded per chunk of 2**22 elements with
  ``SeedSequence([config_seed, crc32(tensor_name), chunk_index])``.  The result does not
  depend on how many threads generate it.
* Projection, embedding and output weights are N(0, 0.02) (0.02 is the standard
  deviation); norm weights are 1 + N(0, 0.1); activations are N(0, 1).
* bf16 tensors are the float32 draws rounded to nearest-even on the bit pattern and kept
  as ``uint16``; fp32 tensors are the float32 draws.
* Token ids are uniform over [0, vocab) from PCG64 seeded with
  ``SeedSequence([config_seed, crc32("tokens")])``.

Tensor names follow the checkpoint keys printed in the article "250 lines of code to build
Llama 3 from scratch" (ai02.cc), section 下载并读取模型权重 (loading the weights).
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class ModelSpec:
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_hidden: int
    vocab_size: int
    norm_eps: float = 1e-5
    rope_theta: float = 500000.0
    dtype: str = "bf16"  # storage type of weights: "bf16" or "f32"


# The five workloads the pages' subject is measured on.
TINY = ModelSpec(dim=64, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=16, ffn_hidden=192,
                 vocab_size=256, dtype="f32")
LLAMA3_8B = ModelSpec(dim=4096, n_layers=32, n_heads=32, n_kv_heads=8, head_dim=128,
                      ffn_hidden=14336, vocab_size=128256, dtype="bf16")
LLAMA3_8B_ONE_LAYER = dataclasses.replace(LLAMA3_8B, n_layers=1)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_chunk(seed: int, key: int, chunk: int, n: int) -> np.ndarray:
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, chunk])))
    return gen.standard_normal(n, dtype=np.float32)


def normal(seed: int, name: str, shape, mean: float = 0.0, std: float = 1.0,
           dtype: str = "f32", threads: int | None = None) -> np.ndarray:
    """Seeded N(mean, std) tensor of ``shape``: float32, or bf16 bits (uint16) if dtype == "bf16"."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    key = zlib.crc32(name.encode())
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = _normal_chunk(seed, key, c, hi - lo)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    workers = threads or _threads()
    if n_chunks <= 1 or workers == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(min(workers, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def tokens(seed: int, batch: int, seq: int, vocab_size: int) -> np.ndarray:
    """Seeded uniform token ids in [0, vocab_size), int32 [batch, seq]."""
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(b"tokens")])))
    return gen.integers(0, vocab_size, size=(batch, seq), dtype=np.int64).astype(np.int32)


def layer_weight_specs(spec: ModelSpec, layer: int):
    """(name, shape, mean, std) of one layer's weights, [out, in] as in the checkpoint."""
    D, H, G, d, F = spec.dim, spec.n_heads, spec.n_kv_heads, spec.head_dim, spec.ffn_hidden
    p = f"layers.{layer}."
    return [
        (p + "attention_norm.weight", (D,), 1.0, 0.1),
        (p + "attention.wq.weight", (H * d, D), 0.0, 0.02),
        (p + "attention.wk.weight", (G * d, D), 0.0, 0.02),
        (p + "attention.wv.weight", (G * d, D), 0.0, 0.02),
        (p + "attention.wo.weight", (D, H * d), 0.0, 0.02),
        (p + "ffn_norm.weight", (D,), 1.0, 0.1),
        (p + "feed_forward.w1.weight", (F, D), 0.0, 0.02),
        (p + "feed_forward.w3.weight", (F, D), 0.0, 0.02),
        (p + "feed_forward.w2.weight", (D, F), 0.0, 0.02),
    ]


def global_weight_specs(spec: ModelSpec):
    D, V = spec.dim, spec.vocab_size
    return [
        ("tok_embeddings.weight", (V, D), 0.0, 0.02),
        ("norm.weight", (D,), 1.0, 0.1),
        ("output.weight", (V, D), 0.0, 0.02),
    ]


def weight_specs(spec: ModelSpec):
    out = list(global_weight_specs(spec))
    for l in range(spec.n_layers):
        out += layer_weight_specs(spec, l)
    return out


class SyntheticWeights:
    """Lazily generated, memoised weight tensors in storage form (uint16 bf16 bits or float32).

    ``stored(name)`` gives the storage form that the GPU receives; ``as_float(name, dtype)``
    gives the exact widening that the oracle consumes.  ``cache=False`` regenerates on
    every request, which keeps host memory bounded at the 8B shape.
    """

    def __init__(self, spec: ModelSpec, seed: int, cache: bool = True):
        self.spec = spec
        self.seed = seed
        self.cache = cache
        self._specs = {n: (s, m, sd) for n, s, m, sd in weight_specs(spec)}
        self._mem: dict[str, np.ndarray] = {}

    def names(self):
        return list(self._specs)

    def shape(self, name: str):
        return self._specs[name][0]

    def stored(self, name: str) -> np.ndarray:
        if name in self._mem:
            return self._mem[name]
        shape, mean, std = self._specs[name]
        a = normal(self.seed, name, shape, mean=mean, std=std, dtype=self.spec.dtype)
        if self.cache:
            self._mem[name] = a
        return a

    def as_float(self, name: str, dtype=np.float64) -> np.ndarray:
        a = self.stored(name)
        f = bf16_bits_to_f32(a) if self.spec.dtype == "bf16" else a
        return f.astype(dtype, copy=False)

    def drop(self, prefix: str = "") -> None:
        for k in [k for k in self._mem if k.startswith(prefix)]:
            del self._mem[k]


class FloatView:
    """Mapping name -> float array over a SyntheticWeights, in the dtype the oracle asks for."""

    def __init__(self, weights: SyntheticWeights, dtype=np.float64):
        self.w = weights
        self.dtype = dtype

    def __getitem__(self, name: str) -> np.ndarray:
        return self.w.as_float(name, self.dtype)
