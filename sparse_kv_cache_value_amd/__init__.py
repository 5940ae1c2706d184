"""Sparse KV-cache refresh for bidirectional diffusion LLMs on MI355X (gfx950).

The compute path lives in the HIP/C++ shared library ``libdllm.so`` (built from
``csrc/``); :mod:`.binding` exposes its C-ABI entry points under the same names.
Submodules are imported lazily so that the seeded input generator can be used
without loading the native library.
"""

__all__ = ["configs", "inputs", "binding", "runtime"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
