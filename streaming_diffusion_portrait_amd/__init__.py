"""MI355X-native hot path of the PersonaLive streaming pyramid denoiser.

The computation lives in ``libpl.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/pl.h``).  ``binding`` is a thin ctypes layer with
the same names; PyTorch supplies device memory and streams only.  ``inputs``
draws the seeded synthetic workloads.

The binding is imported lazily so that ``inputs`` can be used without torch.
"""

import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
