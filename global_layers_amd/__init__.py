"""MI355X (gfx950) Gemma 3 attention-block forward behind a C ABI.

``global_layers_amd.lib`` is the ctypes binding of ``libgemma3_attn.so``
(prefill and decode entry points); ``global_layers_amd.build`` compiles it.
"""

__all__ = ["lib", "build"]
