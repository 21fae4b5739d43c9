"""Grouped-query attention (MHA / GQA / MQA) prefill and KV-cached decode for MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (``include/gqa.h``,
``libgqa.so``).  ``ops`` is a thin ctypes binding with the C entry points'
names; PyTorch supplies device memory and the current HIP stream only.
``inputs`` draws the seeded synthetic workloads.
"""

__all__ = ["inputs", "ops"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
