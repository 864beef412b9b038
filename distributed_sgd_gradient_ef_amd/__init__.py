"""MI355X-native PowerSGD rank-r gradient compression with error feedback.

The compute path is the C-ABI library ``libpsgd.so`` (hand-written gfx950 HIP kernels);
``distributed_sgd_gradient_ef_amd.psgd`` is its thin ctypes binding.
"""
