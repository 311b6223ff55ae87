"""quant_mat_vec_amd: quantized matrix-vector products (MMVQ) for MI355X.

The compute path is the HIP library ``libqmv.so`` (built from ``csrc/``);
``qmv`` is its thin ctypes binding.  Importing the package loads nothing: the
library is opened on the first call and a missing build raises at once.
"""
