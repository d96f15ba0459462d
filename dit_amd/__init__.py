"""dit_amd: fixed-m ("const-max") attention forward for MI355X (gfx950).

The compute path is the C-ABI library ``libfixedm.so`` (HIP kernels under ``csrc/``,
declared in ``include/fixedm.h``); ``dit_amd.fixedm`` is its thin ctypes binding.
Importing this package does not load the library; ``dit_amd.fixedm.lib()`` does.
"""
__all__ = ["fixedm", "workloads"]
