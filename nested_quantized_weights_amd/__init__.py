"""nested_quantized_weights_amd -- MI355X-native nested-weight speculative round.

BitNest-style self-speculative decoding: the draft and the target share one
dual-plane (4-bit base + 4-bit refinement) weight copy and one nested KV
cache. The hot path is hand-written HIP for gfx950 behind the C ABI declared
in include/nestspec.h. ``nested_quantized_weights_amd.nestspec`` is the thin
Python binding (ctypes + torch device memory and streams).

Importing the package loads nothing. The HIP library is loaded on the first
use of the binding, which raises if the library is missing.
"""

_BINDING = ("nest_pack", "nest_act_quant", "draft_gemv", "verify_gemm", "verify_accept",
            "kv_nest_pack", "kv_nest_attend", "NestError", "NestKV", "library_path")

__all__ = list(_BINDING) + ["synth"]


def __getattr__(name):
    if name in _BINDING:
        from . import nestspec

        return getattr(nestspec, name)
    raise AttributeError(name)
