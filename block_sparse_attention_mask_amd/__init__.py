"""Block-sparse (optionally permuted) softmax attention forward on MI355X.

The compute path is the HIP library ``libbsattn.so`` (C ABI in
``include/bsattn.h``); this package holds its thin Python binding
(``api``), the composition of one pass of the path (``pipeline``) and the
pair/FLOP accounting (``metrics``).  The seeded synthetic workloads used by
the tests and the benchmark live outside the package (``synth.py`` at the
repository root).
"""
from ._lib import BsaError, EXPORTS, LIB_PATH  # noqa: F401
from .api import (attn_fwd, build_csr, csr_count, csr_fill, device_cus, perm_from_labels,  # noqa: F401
                  permute_rows, schedule, unpermute_rows, version)
