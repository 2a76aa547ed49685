"""Memory-bounded MoE layer for AMD Instinct MI355X (gfx950).

The layer lives in ``libmoebound.so`` (C ABI in ``include/moebound.h``);
``binding`` marshals torch tensors to it.  Import of this package has no side
effects: the library is loaded on first use.
"""

__all__ = ["binding"]
