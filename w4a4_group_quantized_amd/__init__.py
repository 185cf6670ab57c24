"""MI355X-native pure W4A4 group-quantized GEMM (APEX4-style), HIP/gfx950.

Importing the package loads nothing; ``w4a4_group_quantized_amd.apex4`` loads
the C-ABI library ``libapex4.so`` built from ``csrc/``.
"""
__all__ = ["inputs"]
