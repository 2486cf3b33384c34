"""Affine autoregressive-flow block (STARFlow-V) on AMD MI355X: HIP kernels
for gfx950 behind the C ABI in include/af.h, with a thin ctypes binding
(``autoregressive_normalizing_flow_amd.binding``, imported on first use so
that the seeded input module ``synth`` works without the built library)."""
import importlib

__all__ = ["synth", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
