"""HiFA4-style MXFP4 FlashAttention for MI355X (gfx950).

The compute path is the C-ABI library ``libhifa4.so`` built from ``csrc/``;
``binding`` marshals torch tensors into it.  ``workloads`` draws the seeded
synthetic inputs.
"""
