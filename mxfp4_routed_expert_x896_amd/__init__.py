"""MXFP4 routed-expert MoE layer for AMD Instinct MI355X (gfx950).

The product is the C-ABI library libmoe_mxfp4.so (include/moe_mxfp4.h),
built from csrc/ by `python -m mxfp4_routed_expert_x896_amd.build`;
`binding` is its thin ctypes wrapper.  Import `binding` explicitly: importing
this package alone loads nothing.
"""

__all__ = ["binding", "build"]
