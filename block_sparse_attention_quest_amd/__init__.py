"""MI355X-native PRR (predict, reuse, repair) decode hot path.

The compute lives in the C-ABI library libprr.so (hand-written HIP for gfx950, sources under csrc/);
`binding` marshals torch device tensors into its entry points.  Importing the binding on a machine
without the built library raises; there is no CPU fallback.
"""
__all__ = ["workloads"]
