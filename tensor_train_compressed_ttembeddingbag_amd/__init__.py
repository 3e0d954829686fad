"""TT-EmbeddingBag for AMD MI355X (gfx950).

An EmbeddingBag whose table is never stored: each requested row is rebuilt from
three Tensor-Train cores and sum-pooled per bag, with a backward pass that updates
the cores in place (fused sparse SGD) and an HBM cache of decompressed hot rows.
The compute runs in hand-written HIP kernels behind the C ABI in
``include/tt_bag.h`` (``libttbag.so``); ``abi`` is the thin ctypes binding and
``module`` a small torch.nn.Module on top of it.

Importing this package does not load the HIP library; the first call into
``abi`` does, and raises if the library has not been built.
"""
from . import metrics, workloads  # noqa: F401

__all__ = ["metrics", "workloads", "abi", "module"]


def __getattr__(name):
    if name in ("abi", "module"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
