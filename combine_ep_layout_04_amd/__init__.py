"""MI355X-native MoE token layout, dispatch and combine (one device's share).

The work runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/ep.h`` (``libep.so``); :mod:`combine_ep_layout_04_amd.ep` is the
Python binding with the same names (``ep_layout``, ``ep_dispatch``,
``ep_combine``).  :mod:`combine_ep_layout_04_amd.inputs` draws the seeded
synthetic workloads.  Importing the package loads nothing; the library is
loaded on first use and a missing library raises.
"""

__all__ = ["ep_layout", "ep_dispatch", "ep_combine", "EpError"]


def __getattr__(name):
    if name in __all__:
        from . import ep
        return getattr(ep, name)
    raise AttributeError(name)
