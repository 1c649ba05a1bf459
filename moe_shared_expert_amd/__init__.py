"""MI355X-native shared-expert SwiGLU MLP (Kimi-K3 shapes) behind a C-ABI.

The compute lives in ``libsmlp.so`` (hand-written HIP for gfx950).  This
package only marshals torch tensors (device memory) and the current HIP stream
into that library; it is loaded on first use.
"""
from . import roofline  # noqa: F401


def __getattr__(name):
    # The binding is imported lazily so that host-only users (byte accounting,
    # CPU tests) do not need the HIP runtime.
    if name in ("binding",):
        import importlib
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
