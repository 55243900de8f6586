"""MI355X-native slot-indexed KV cache and batched decode-attention step.

The product is the C ABI in ``include/slot_kv.h`` (``libslot_kv.so``, HIP for
gfx950); ``binding`` is its thin ctypes layer and ``workloads`` the seeded
synthetic inputs.  ``binding`` loads on first use so that the input
generators import without the library; using any library name when the
library is not built raises ImportError.
"""
import importlib

__all__ = ["binding", "workloads", "SlotKV", "SlotKVError"]


def __getattr__(name):
    if name in ("SlotKV", "SlotKVError"):
        return getattr(importlib.import_module(".binding", __name__), name)
    raise AttributeError(name)
