"""Paged, varlen, causal attention with a relative-position bias for MI355X.

The compute runs in ``librpa.so`` (hand-written HIP for gfx950) behind a C ABI;
``relative_bias_amd.binding`` marshals torch tensors into it.  Import the
binding explicitly; this package import loads nothing native.
"""
__all__ = ["binding", "workloads"]
