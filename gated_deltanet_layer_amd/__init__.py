"""gated_deltanet_layer_amd: the gated DeltaNet token mixer on MI355X (gfx950).

The compute lives in a HIP C-ABI library (``libgdn.so``, declared in
``include/gdn.h``). ``gated_deltanet_layer_amd.binding`` is its thin Python
binding; importing the package itself loads nothing, so that the seeded
workload generator (``workloads``) can be used without the library.
"""

__all__ = ["workloads", "binding"]
