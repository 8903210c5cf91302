"""Group-scaled 1-bit (Q1_0_g128) and ternary (g128) y = W.x for MI355X.

The compute path is the HIP library ``liblowbit.so`` built from ``csrc/``;
``bit_matmul_lowbit_amd.lowbit`` is its thin ctypes binding.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""
__all__ = ["lowbit", "synth"]
