"""MI355X-native OmniMoE routed-branch forward.

The compute path is the HIP library `libomni.so` (built from csrc/ for
gfx950); `atomic_expert_routing_amd.omni` is a thin ctypes binding over its
C ABI.  Importing the package loads nothing: the library is opened on first
use and a missing or stale build raises instead of falling back.
"""

__all__ = ["omni", "synth"]
