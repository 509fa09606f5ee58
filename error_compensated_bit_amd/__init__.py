"""MI355X (gfx950) library for the data-parallel hot path of 1-bit Adam.

The kernels live in libonebit.so (C ABI in include/onebit.h); `onebit` is its
Python binding, `optimizer` sequences its calls into 1-bit Adam's two phases,
`workloads` builds seeded synthetic inputs.  The binding is
loaded on first use so that the input generators import without a GPU.
"""
import importlib


def __getattr__(name):
    if name.startswith("__") or name in ("onebit", "optimizer", "workloads", "build"):
        raise AttributeError(name)
    mod = importlib.import_module(__name__ + ".onebit")
    try:
        return getattr(mod, name)
    except AttributeError:
        raise AttributeError(name) from None
