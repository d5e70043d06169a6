"""TokenGate gated prefill on MI355X (gfx950).

The compute path lives in ``libtg.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/tg.h``); :mod:`learned_token_pruning_tg_amd.tg` is
its thin Python binding.  Importing the package does not load the library; the
first call into :mod:`.tg` does, and raises if it has not been built.
"""

__all__ = ["tg", "inputs"]


def __getattr__(name):
    if name in ("tg", "inputs"):
        import importlib

        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
