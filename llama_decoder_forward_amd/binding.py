"""ctypes binding of ``libllama_mi355x.so`` (argument marshalling only).

Every step of the forward pass runs in the HIP library; this module only builds the C
structs, passes device pointers of torch tensors and the current HIP stream, and raises
``LlamaError`` on a non-OK status.  PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libllama_mi355x.so")

LLAMA_BF16, LLAMA_F32 = 0, 1
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "SHAPE", -3: "CAPACITY", -4: "DTYPE", -5: "HIP",
          -6: "ALLOC"}


class LlamaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class LlamaConfig(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_hidden", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("max_batch", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class LlamaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w3", "w2")]


class LlamaWeights(ctypes.Structure):
    _fields_ = [("tok_embeddings", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LlamaLayerWeights)),
                ("norm", ctypes.c_void_p), ("output", ctypes.c_void_p)]


EXPORTS = ["llama_kv_cache_bytes", "llama_workspace_bytes", "llama_init_weights", "llama_prefill",
           "llama_prefill_at", "llama_decode_step", "llama_decode_step_noalloc",
           "llama_decode_step_ragged", "llama_generate", "llama_layer_forward",
           "llama_sync_status", "llama_trace_hidden", "llama_free", "llama_last_error",
           "llama_profile_kernel", "llama_profile_read"]

KERNELS = {"none": 0, "qkv": 1, "attention": 2, "wo": 3, "ffn_up": 4, "ffn_down": 5,
           "lm_head": 6, "rmsnorm": 7}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with llama_decoder_forward_amd.build "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.POINTER
    lib.llama_kv_cache_bytes.argtypes = [F(LlamaConfig)]
    lib.llama_kv_cache_bytes.restype = Z
    lib.llama_workspace_bytes.argtypes = [F(LlamaConfig)]
    lib.llama_workspace_bytes.restype = Z
    lib.llama_init_weights.argtypes = [F(LlamaConfig), F(LlamaWeights), P, Z, P, Z, F(P)]
    lib.llama_prefill.argtypes = [P, P, I, I, P, I, P]
    lib.llama_prefill_at.argtypes = [P, P, I, I, I, P, I, P, P]
    lib.llama_decode_step.argtypes = [P, P, I, I, P, P, P]
    lib.llama_decode_step_noalloc.argtypes = [P, P, I, I, P, P, P]
    lib.llama_decode_step_ragged.argtypes = [P, P, I, P, P, P, P]
    lib.llama_generate.argtypes = [P, P, I, I, I, P, P, P]
    lib.llama_layer_forward.argtypes = [P, I, P, P, I, I, I, P]
    lib.llama_sync_status.argtypes = [P, P]
    lib.llama_trace_hidden.argtypes = [P, P, I]
    lib.llama_profile_kernel.argtypes = [P, ctypes.c_int]
    lib.llama_profile_read.argtypes = [P, F(ctypes.c_double), F(ctypes.c_int32)]
    lib.llama_free.argtypes = [P]
    lib.llama_free.restype = None
    lib.llama_last_error.argtypes = []
    lib.llama_last_error.restype = ctypes.c_char_p
    for fn in ("llama_init_weights", "llama_prefill", "llama_prefill_at", "llama_decode_step",
               "llama_decode_step_noalloc", "llama_decode_step_ragged", "llama_generate",
               "llama_layer_forward", "llama_sync_status", "llama_trace_hidden",
               "llama_profile_kernel", "llama_profile_read"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        raise LlamaError(status, load_library().llama_last_error().decode())


def make_config(spec, max_batch: int, max_seq: int, max_tokens: int) -> LlamaConfig:
    return LlamaConfig(spec.dim, spec.n_layers, spec.n_heads, spec.n_kv_heads, spec.head_dim,
                       spec.ffn_hidden, spec.vocab_size, spec.norm_eps, spec.rope_theta,
                       max_batch, max_seq, max_tokens,
                       LLAMA_BF16 if spec.dtype == "bf16" else LLAMA_F32)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def upload_weights(synth, device="cuda") -> dict:
    """Copy every tensor of a synthetic.SyntheticWeights to the device, in storage dtype."""
    out = {}
    for name in synth.names():
        a = synth.stored(name)
        if synth.spec.dtype == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out[name] = t.to(device, non_blocking=False)
        if not synth.cache:
            del a
    return out


class Model:
    """A model handle over caller-owned device buffers (weights, KV cache, workspace)."""

    def __init__(self, spec, weights: dict, max_batch: int, max_seq: int, max_tokens: int,
                 device="cuda"):
        self.lib = load_library()
        self.spec = spec
        self.cfg = make_config(spec, max_batch, max_seq, max_tokens)
        self.weights = weights  # keep the tensors alive
        kvb = self.lib.llama_kv_cache_bytes(ctypes.byref(self.cfg))
        wsb = self.lib.llama_workspace_bytes(ctypes.byref(self.cfg))
        if kvb == 0 or wsb == 0:
            raise LlamaError(-2, f"invalid config: {self.lib.llama_last_error().decode()}")
        self.kv = torch.empty(kvb, dtype=torch.uint8, device=device)
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device=device)
        L = spec.n_layers
        self._layers = (LlamaLayerWeights * L)()
        for l in range(L):
            p = f"layers.{l}."
            self._layers[l] = LlamaLayerWeights(*[
                _ptr(weights[p + n]) for n in
                ("attention_norm.weight", "attention.wq.weight", "attention.wk.weight",
                 "attention.wv.weight", "attention.wo.weight", "ffn_norm.weight",
                 "feed_forward.w1.weight", "feed_forward.w3.weight", "feed_forward.w2.weight")])
        self._w = LlamaWeights(_ptr(weights["tok_embeddings.weight"]), self._layers,
                               _ptr(weights["norm.weight"]), _ptr(weights["output.weight"]))
        h = ctypes.c_void_p()
        check(self.lib.llama_init_weights(ctypes.byref(self.cfg), ctypes.byref(self._w),
                                          _ptr(self.kv), kvb, _ptr(self.ws), wsb, ctypes.byref(h)))
        self.handle = h
        self.device = device
        self.seq_stride = (max_seq + 63) // 64 * 64

    # -------------------------------------------------------------- calls
    def prefill(self, tokens: torch.Tensor, all_positions: bool = False, logits=None, stream=None,
                start_pos: int = 0, want_next: bool = False):
        """Prefill [B, S] tokens at positions start_pos.. (llama_prefill / llama_prefill_at).
        Returns the logits, or (logits, next tokens [B]) with want_next."""
        B, S = tokens.shape
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        V = self.spec.vocab_size
        if logits is None:
            shape = (B, S, V) if all_positions else (B, V)
            logits = torch.empty(shape, dtype=torch.float32, device=self.device)
        nxt = torch.empty(B, dtype=torch.int32, device=self.device) if want_next else None
        if start_pos == 0 and not want_next:
            check(self.lib.llama_prefill(self.handle, _ptr(tokens), B, S, _ptr(logits),
                                         int(all_positions), _stream(stream)))
        else:
            check(self.lib.llama_prefill_at(self.handle, _ptr(tokens), B, S, start_pos,
                                            _ptr(logits), int(all_positions), _ptr(nxt),
                                            _stream(stream)))
        return (logits, nxt) if want_next else logits

    def decode_step(self, tokens: torch.Tensor, pos: int, want_logits: bool = True,
                    next_tokens=None, logits=None, stream=None):
        B = tokens.shape[0]
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        if next_tokens is None:
            next_tokens = torch.empty(B, dtype=torch.int32, device=self.device)
        if want_logits and logits is None:
            logits = torch.empty((B, self.spec.vocab_size), dtype=torch.float32, device=self.device)
        check(self.lib.llama_decode_step(self.handle, _ptr(tokens), B, pos,
                                         _ptr(logits) if want_logits else None,
                                         _ptr(next_tokens), _stream(stream)))
        return next_tokens, (logits if want_logits else None)

    def decode_step_noalloc(self, tokens: torch.Tensor, pos: int, want_logits: bool = True,
                            next_tokens=None, logits=None, stream=None):
        """llama_decode_step_noalloc: decode_step with its scratch in the library's static
        array (no workspace scratch)."""
        B = tokens.shape[0]
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        if next_tokens is None:
            next_tokens = torch.empty(B, dtype=torch.int32, device=self.device)
        if want_logits and logits is None:
            logits = torch.empty((B, self.spec.vocab_size), dtype=torch.float32, device=self.device)
        check(self.lib.llama_decode_step_noalloc(self.handle, _ptr(tokens), B, pos,
                                                 _ptr(logits) if want_logits else None,
                                                 _ptr(next_tokens), _stream(stream)))
        return next_tokens, (logits if want_logits else None)

    def trace_hidden(self, max_rows: int | None):
        """Record the residual stream of later calls (llama_trace_hidden) into a new tensor
        [n_layers + 1, max_rows, dim], returned; None stops recording."""
        if max_rows is None:
            check(self.lib.llama_trace_hidden(self.handle, None, 0))
            self._trace = None
            return None
        buf = torch.zeros((self.spec.n_layers + 1, max_rows, self.spec.dim), dtype=torch.float32,
                          device=self.device)
        check(self.lib.llama_trace_hidden(self.handle, _ptr(buf), max_rows))
        self._trace = buf  # keep it alive while recorded into
        return buf

    def decode_step_ragged(self, tokens: torch.Tensor, positions: torch.Tensor,
                           want_logits: bool = True, next_tokens=None, logits=None, stream=None):
        """One decode step with a position per sequence (device int32 [B])."""
        B = tokens.shape[0]
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        assert positions.dtype == torch.int32 and positions.is_contiguous() and positions.is_cuda
        assert positions.shape == (B,)
        if next_tokens is None:
            next_tokens = torch.empty(B, dtype=torch.int32, device=self.device)
        if want_logits and logits is None:
            logits = torch.empty((B, self.spec.vocab_size), dtype=torch.float32, device=self.device)
        check(self.lib.llama_decode_step_ragged(self.handle, _ptr(tokens), B, _ptr(positions),
                                                _ptr(logits) if want_logits else None,
                                                _ptr(next_tokens), _stream(stream)))
        return next_tokens, (logits if want_logits else None)

    def generate(self, tokens: torch.Tensor, pos: int, n_steps: int, want_logits: bool = False,
                 out_tokens=None, stream=None):
        B = tokens.shape[0]
        if out_tokens is None:
            out_tokens = torch.empty((n_steps, B), dtype=torch.int32, device=self.device)
        logits = (torch.empty((n_steps, B, self.spec.vocab_size), dtype=torch.float32,
                              device=self.device) if want_logits else None)
        check(self.lib.llama_generate(self.handle, _ptr(tokens), B, pos, n_steps,
                                      _ptr(out_tokens), _ptr(logits), _stream(stream)))
        return out_tokens, logits

    def layer_forward(self, layer: int, x_in: torch.Tensor, start_pos: int = 0, x_out=None,
                      stream=None):
        B, S, D = x_in.shape
        assert x_in.dtype == torch.float32 and x_in.is_contiguous()
        if x_out is None:
            x_out = torch.empty_like(x_in)
        check(self.lib.llama_layer_forward(self.handle, layer, _ptr(x_in), _ptr(x_out), B, S,
                                           start_pos, _stream(stream)))
        return x_out

    def profile_kernel(self, kind: str):
        """Time every launch of one kernel class with HIP events (kind in KERNELS)."""
        check(self.lib.llama_profile_kernel(self.handle, KERNELS[kind]))

    def profile_read(self):
        """(total milliseconds, launches) timed since profile_kernel; resets the counts."""
        ms, n = ctypes.c_double(), ctypes.c_int32()
        check(self.lib.llama_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def sync_status(self, stream=None):
        check(self.lib.llama_sync_status(self.handle, _stream(stream)))

    # -------------------------------------------------------------- cache views (tests)
    def _elem(self):
        return torch.bfloat16 if self.spec.dtype == "bf16" else torch.float32

    def kv_packed(self) -> bool:
        """Whether the library keeps this model's KV cache in its packed layout: bf16 with
        head_dim 128 and at most 16 query heads per KV head dividing 128, i.e. exactly the
        shapes whose attention runs on the matrix-core kernels."""
        c = self.cfg
        group = c.n_heads // c.n_kv_heads
        return (self.spec.dtype == "bf16" and c.head_dim == 128 and group <= 16
                and 128 % group == 0)

    def cache_k(self, layer: int) -> torch.Tensor:
        """K cache of one layer as [max_batch, G, seq_stride, d] (a view of the plain layout,
        or a reordered copy of the packed one)."""
        c = self.cfg
        n = c.max_batch * c.n_kv_heads * self.seq_stride * c.head_dim
        es = 2 if self.spec.dtype == "bf16" else 4
        base = layer * 2 * n * es
        raw = self.kv[base:base + n * es].view(self._elem())
        if not self.kv_packed():
            return raw.view(c.max_batch, c.n_kv_heads, self.seq_stride, c.head_dim)
        # packed: within a 64-position block, [t/2][t%2][jj][col/4][kq][col%4][e] holds key
        # r = 32 (t/2) + 8 (col/4) + 4 (t%2) + col%4, dimension 32 jj + 8 kq + e
        blk = raw.view(c.max_batch, c.n_kv_heads, self.seq_stride // 64, 2, 2, 4, 4, 4, 4, 8)
        return blk.permute(0, 1, 2, 3, 6, 4, 8, 5, 7, 9).reshape(
            c.max_batch, c.n_kv_heads, self.seq_stride, c.head_dim)

    def cache_v(self, layer: int) -> torch.Tensor:
        """V cache of one layer as [max_batch, G, seq_stride, d] (from the stored layout:
        transposed within blocks of 64 positions, [b][g][pos/64][d][64], or packed)."""
        c = self.cfg
        n = c.max_batch * c.n_kv_heads * self.seq_stride * c.head_dim
        es = 2 if self.spec.dtype == "bf16" else 4
        base = (layer * 2 + 1) * n * es
        raw = self.kv[base:base + n * es].view(self._elem())
        if not self.kv_packed():
            vt = raw.view(c.max_batch, c.n_kv_heads, self.seq_stride // 64, c.head_dim, 64)
            return vt.permute(0, 1, 2, 4, 3).reshape(c.max_batch, c.n_kv_heads,
                                                     self.seq_stride, c.head_dim)
        # packed: within a 64-position block, [dt][j][kq][col][e] holds dimension 16 dt + col
        # of key r = 32 j + 8 kq + e
        blk = raw.view(c.max_batch, c.n_kv_heads, self.seq_stride // 64, 8, 2, 4, 16, 8)
        return blk.permute(0, 1, 2, 4, 5, 7, 3, 6).reshape(
            c.max_batch, c.n_kv_heads, self.seq_stride, c.head_dim)

    def free(self):
        if getattr(self, "handle", None):
            self.lib.llama_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
