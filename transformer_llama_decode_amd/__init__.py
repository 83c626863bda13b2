"""MI355X (gfx950) fp32 Llama-2-architecture decode: HIP kernels behind a C ABI.

    from transformer_llama_decode_amd import LlamaDecoder, WORKLOADS
"""
from .configs import ModelConfig, Workload, WORKLOADS, TINY, TINY_UNTIED, SMALL  # noqa: F401


def __getattr__(name):
    # the HIP library is only loaded when the model API is used
    if name in ("LlamaDecoder", "arena_bytes", "synth_prompt"):
        from . import model
        return getattr(model, name)
    raise AttributeError(name)
