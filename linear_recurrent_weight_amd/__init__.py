"""MI355X-native Falcon fast-weight forward pass and Falcon-1 backward pass
(HIP kernels behind a C ABI).

Importing the package does not load the native library; ``falcon_fwd`` and
friends load ``libfalcon.so`` on first use and raise if it is missing.
"""
__all__ = ["fwd", "bwd", "FalconState", "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import falcon
        return getattr(falcon, name)
    raise AttributeError(name)
