"""Exact tiled attention for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/fa.h``); :mod:`.binding` marshals PyTorch
tensors into it.  :mod:`.inputs` builds seeded synthetic workloads and
:mod:`.metrics` counts algorithmic work.
"""

__all__ = ["binding", "inputs", "metrics"]


def __getattr__(name):
    # The binding loads the HIP library; import it only when asked for.
    if name in ("binding", "fa_fwd", "fa_decode", "fa_decode_workspace_size", "fa_status_string"):
        import importlib
        mod = importlib.import_module(f"{__name__}.binding")
        return mod if name == "binding" else getattr(mod, name)
    raise AttributeError(name)
