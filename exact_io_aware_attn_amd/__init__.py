"""MI355X-native exact attention forward (tiled, online softmax, split-D).

The compute path is the C-ABI library ``libattn.so`` built from the HIP
sources in ``csrc/`` for gfx950; ``attn`` is its thin ctypes binding.  The
binding is imported lazily so that input generation works on machines
without a GPU; calling into it without the built library raises.
"""
__version__ = "0.1.0"


def __getattr__(name):
    if name in ("fwd", "fwd_fp8", "lib", "AttnError"):
        from . import attn

        return getattr(attn, name)
    raise AttributeError(name)
