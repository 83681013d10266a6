"""MI355X-native verify step of speculative decoding (HIP for gfx950).

The compute path lives in the C-ABI library built from ``csrc/`` (see
``include/spec_verify.h``); ``binding`` marshals torch tensors to it.  The
binding is imported lazily so that the input generators in ``workloads`` work
on machines without a built library.
"""


def __getattr__(name):
    if name in ("binding",):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
