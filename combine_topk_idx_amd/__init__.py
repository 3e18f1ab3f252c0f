"""MoE token dispatch and combine for AMD Instinct MI355X (gfx950).

The work is done by the C-ABI library ``libep.so`` (HIP kernels for gfx950,
sources under ``csrc/``, declarations in ``include/ep.h``).  ``ep`` is the
thin ctypes binding with the same function names; importing it loads the
library and raises if it is missing -- there is no CPU fallback.

``workloads`` draws the seeded synthetic inputs used by the tests and the
benchmark; it is importable without the library.
"""

__all__ = ["ep", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
