"""GDN-CPR for MI355X: the Chunkwise-Parallel Recurrent Gated DeltaNet hot path as a C-ABI
HIP library (``libgdn_cpr.so``) with a thin ctypes binding.

Importing the package loads nothing; the native library is loaded on first use through
:mod:`bitwise_consistent_linear_amd.api`.
"""
