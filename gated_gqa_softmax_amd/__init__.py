"""Gated grouped-query causal attention (forward pass) for MI355X / gfx950.

The computation runs in hand-written HIP kernels inside ``libga.so`` behind
the C ABI declared in ``include/ga.h``; ``gated_gqa_softmax_amd.api`` binds
each entry point by the same name. ``inputs`` draws the seeded synthetic
workloads and ``accounting`` gives the algorithmic flop and byte counts.
"""
__all__ = ["api", "inputs", "accounting"]
