"""TokenGate gated prefill on MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libtokengate.so`` (built from ``csrc/``); ``binding``
marshals torch device tensors into it. ``workloads`` draws the seeded
synthetic inputs. Importing the package itself loads nothing.
"""
__all__ = ["binding", "workloads", "build"]
