"""sparq24 for MI355X: online 2:4 prune-and-compress, dense quantizers and the
energy reductions that score them (Qin, "Is 2:4 Sparsity Still Worth It?").

The compute lives in ``libsparq24.so`` (HIP kernels for gfx950 behind a C
ABI, see ``include/sparq24.h``); :mod:`.binding` marshals torch tensors into
it.  Build with ``python -m pruning_quantization_amd.build``.
"""
from .binding import (  # noqa: F401
    Sparq24Error,
    SYMBOLS,
    bits_per_element,
    col_l2norm,
    copy,
    dense_gemm,
    describe,
    error_energy,
    fp8_gemm,
    hadamard,
    lib,
    operator_error,
    predict_R,
    predict_R_noalloc,
    prune_compress,
    prune_compress_pairs48,
    predict_R_pairs48,
    predict_R_rot,
    prune_quantize,
    prune_quantize_pairs48,
    prune_quantize_rot,
    qspec,
    quantize,
    quantize_rot,
    sparse_gemm,
    version,
)
