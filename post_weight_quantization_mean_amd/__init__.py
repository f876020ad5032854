"""AWQ activation-aware INT4 scale search and packing on MI355X (gfx950).

The compute path is the C-ABI library ``libawq.so`` (hand-written HIP kernels); the Python
layer in :mod:`post_weight_quantization_mean_amd.awq` only marshals arguments.  Importing
this package does not load the library; ``stats``/``search``/``pack`` load it on first use
and raise if it has not been built.
"""

__all__ = ["stats", "search", "pack", "search_workspace_bytes", "stats_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import awq
        return getattr(awq, name)
    raise AttributeError(name)
