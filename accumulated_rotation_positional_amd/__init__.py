"""Causal attention with accumulated SO(2) rotations on AMD MI355X (gfx950).

The compute path is the C-ABI library ``libarp.so`` (hand-written HIP kernels);
``binding`` marshals torch device tensors into it.  ``workloads`` builds the
seeded synthetic inputs.
"""
