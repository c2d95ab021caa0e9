"""libssmscan: the Mamba selective state-space scan (S6) for MI355X (gfx950).

The compute path is the C-ABI shared library ``libssmscan.so`` (hand-written HIP
kernels); ``selective_state_space_32_amd.ssmscan`` is its thin ctypes binding taking
torch tensors.  ``selective_state_space_32_amd.inputs`` builds seeded synthetic
workloads.  The binding is imported lazily so that the input generator can be used on
machines without a GPU.
"""
import importlib

__all__ = ["scan_fwd", "step", "workspace_bytes"]


def __getattr__(name):
    if name in ("scan_fwd", "step", "workspace_bytes"):
        return getattr(importlib.import_module(__name__ + ".ssmscan"), name)
    raise AttributeError(name)
