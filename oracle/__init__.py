"""CPU oracle for online 2:4 prune-and-compress, the dense quantizers it is
compared against, and the energy reductions that score the two.

TEST INFRASTRUCTURE ONLY. This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` (to check one small GPU call) and by the
``cpu_baseline`` leg of ``bench.py``. The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package imports nothing from the product path.

Source: Xiuyi Qin, "Is 2:4 Sparsity Still Worth It? Semi-Structured Sparsity
versus Quantization in LLM Inference" (arXiv 2610.28947), as summarised on the
paper-daily.com English page (cited below as "[PD §n]" with the section number
of that page) and in the abstract on weekinpapers.com ("[abstract]").

Everything is plain numpy in fp64. The steps that the method defines in fp32
(per-row and per-block scales, and the scaled value that is rounded to a
code) are evaluated in numpy float32, whose + - * / are IEEE single precision,
so each quantized code is decided in the same precision as on the GPU.
The pages leave several steps open; the readings taken here are listed in the
module docstrings below and in the design notes of the repository.

Parity status: every function here is pinned by CPU tests against values
fixed by the pages, closed forms, library routines or brute force (see
``tests/test_oracle_*.py``). ``col_l2norm`` is pinned by a closed-form check
on constructed columns.
"""
from .reference import (  # noqa: F401
    BF16, F16, F32,
    decode_input,
    score_values,
    select_2of4,
    meta_from_indices,
    indices_from_meta,
    prune_compress,
    decompress,
    pair_scores,
    select_pairs48,
    prune_compress_pairs48,
    decompress_pairs48,
    hadamard_matrix,
    hadamard_scale,
    rotate,
    rotation_exact,
    E4M3_GRID, E2M1_GRID,
    e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode,
    int_rtn_codes,
    row_scale,
    quantize_rows,
    dequantize_rows,
    quantize_mxfp4, dequantize_mxfp4,
    quantize_nvfp4, dequantize_nvfp4,
    quantize_kept,
    dequantize_kept,
    prune_quantize,
    prune_quantize_pairs48,
    dequantize_pruned,
    error_energy,
    predict_R,
    energies_to_R,
    col_l2norm,
    tensor_absmax,
    bits_per_element,
    QSpec,
    Side,
    reconstruct,
    operator_error,
    TINY_AMAX,
)
