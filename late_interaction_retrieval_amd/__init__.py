"""MI355X-native fused late-interaction MaxSim.

score(Q, D) = sum_i max_j <Q_i, D_j>, computed by hand-written gfx950 HIP
kernels behind a C ABI (``include/maxsim.h``); the Python side only marshals
arguments.  Submodules:
  binding  -- ctypes binding with the C entry point names (loads libmaxsim.so)
  inputs   -- seeded synthetic inputs (numpy only)
  build    -- compiles libmaxsim.so for gfx950 with hipcc
"""
__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
