"""MI355X-native Llama-3 decoder forward pass (prefill and KV-cache decode).

The compute runs in the HIP library ``libllama_mi355x.so`` behind the C ABI declared in
``include/llama_mi355x.h``; ``llama_decoder_forward_amd.binding`` marshals arguments to it.
Submodules are imported on demand so that ``synthetic`` can be used without a GPU.
"""
__all__ = ["binding", "synthetic"]
