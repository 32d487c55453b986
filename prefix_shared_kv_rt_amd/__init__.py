"""RadixAttention hot path on AMD Instinct MI355X (gfx950).

``binding`` exposes every C entry point of include/radixrt.h under the same
name (ctypes, argument marshalling only).  ``runtime`` drives a workload
through the tree, the scatter kernel and the two attention kernels.
"""

from . import binding  # noqa: F401
