"""MI355X (gfx950) Gated-Delta-Net recurrence: HIP kernels behind a C ABI (include/gdn.h).

    from gated_deltanet_recurrence_gdn_amd.binding import GDN      # loads libgdn.so
    from gated_deltanet_recurrence_gdn_amd import inputs            # seeded synthetic inputs

The binding is imported on first use so that the input generator stays importable on a
machine where the library has not been built; the binding itself raises if libgdn.so is
missing (there is no fallback implementation).
"""
__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in ("binding", "inputs", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
