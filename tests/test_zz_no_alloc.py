"""The allocation-free predict_R (workspace in the library's static device
array) against the workspace-taking sparq24_predict_R: two calls in a row,
the second on a smaller operand, each compared bit for bit (both run the same
kernels in the same order), plus the size limit checked on the host."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import pruning_quantization_amd as S  # noqa: E402
from pruning_quantization_amd import binding as B  # noqa: E402
from gpu_util import random_raw, to_dev  # noqa: E402


def test_noalloc_matches_workspace_call_twice():
    rng = np.random.default_rng(77)
    big = to_dev(random_raw(rng, (3000, 4096), "bf16"), "bf16")
    kept, dense = ["fp8", ("int", 4), "none"], [("int", 8), "fp8", "nvfp4"]
    print("noalloc call 1: bf16 [3000, 4096], whole operand, 3 pairs", flush=True)
    a = S.predict_R_noalloc(big, kept, dense)
    b = S.predict_R(big, kept, dense)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))
    small = to_dev(random_raw(rng, (700, 1024), "bf16"), "bf16")
    kept2, dense2 = ["fp8", "fp8"], ["mxfp4", ("int", 6)]
    print("noalloc call 2: bf16 [700, 1024], blocks of 128 rows, 2 pairs", flush=True)
    c = S.predict_R_noalloc(small, kept2, dense2, rows_per_block=128)
    d = S.predict_R(small, kept2, dense2, rows_per_block=128)
    torch.cuda.synchronize()
    assert c.shape == (6, 2, 5)
    assert torch.equal(c.view(torch.int64), d.view(torch.int64))
    # the first call's result is untouched by the second call's use of the array
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))


def test_noalloc_rejects_oversized_workspace():
    # rows x columns of fp64 partials beyond the static array: rejected on the
    # host before anything is enqueued (the data pointer is never read)
    c = B.CTensor()
    c.data, c.dtype, c.batch, c.rows, c.k = 0x7F0000000000, B.BF16, 1, 1 << 20, 64
    c.row_stride, c.batch_stride, c.k_stride = 64, (1 << 20) * 64, 1
    arr = (B.CQSpec * 2)(B.qspec("fp8"), B.qspec(("int", 4)))
    st = B.lib().sparq24_predict_R_noalloc(ctypes.byref(c), 0, None, arr, arr, 2, 0,
                                           0x7F0000001000, None)
    assert st == 5  # SPARQ24_ERR_WORKSPACE
