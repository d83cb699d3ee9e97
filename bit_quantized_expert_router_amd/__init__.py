"""MI355X-native routed-MoE expert layer on 2-bit block-quantized weights.

The compute lives in the HIP library ``libmoe_q2.so`` (built from ``csrc/``);
``binding`` marshals torch tensors into its C-ABI.  ``synth`` holds the seeded
input generators.  Importing the package does not load the library; the
binding loads it on first use and raises if it is missing.
"""
__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in ("binding", "synth"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
