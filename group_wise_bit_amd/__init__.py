"""group_wise_bit_amd — group-wise low-bit weight quantization on MI355X (gfx950).

  binding    the Python binding of libgwb.so (C ABI in include/gwb.h); importing it
             raises if the library is not built — there is no fallback path
  workloads  seeded synthetic inputs (no quantization arithmetic)
  _build     hipcc build of libgwb.so

Attributes of the binding (quantize, dequantize, snr, awq_search, ...) are also
reachable from the package itself; the library is loaded on first such access.
"""


def __getattr__(name):
    if name.startswith("__") or name in ("binding", "workloads", "_build"):
        raise AttributeError(name)
    import importlib
    return getattr(importlib.import_module(__name__ + ".binding"), name)
