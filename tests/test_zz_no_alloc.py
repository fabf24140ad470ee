"""bitlinear_forward_noalloc (the allocation-free variant of bitlinear_forward,
scratch in a static device array) through the C ABI: the same bits as
bitlinear_forward on two calls in a row, the second with a smaller input,
over the decode and prefill kernels; sizes past the array are refused."""
import ctypes

import numpy as np
import pytest

import oracle
from ternary_weight_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bl = pytest.importorskip("ternary_weight_amd.bitlinear")

DEV = "cuda"
EPS = inputs.EPS


def _case(seed, M, K, N):
    W = inputs.weight(30, seed, 0, N, K)
    packed, scale = oracle.i2s_pack(W)
    x = inputs.activations(30, seed, 1, M, K)
    nw = inputs.norm_weight(30, seed, 2, K)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return to(x), to(nw), to(packed), scale


def _noalloc(x, nw, pw, scale, N, y):
    """The C ABI call itself (ctypes), on the current stream."""
    M, K = x.shape
    return bl.lib.bitlinear_forward_noalloc(
        x.data_ptr(), None if nw is None else nw.data_ptr(), pw.data_ptr(), ctypes.c_float(scale),
        M, K, N, ctypes.c_float(EPS), y.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("first,second", [
    ((600, 3072, 1024), (40, 1024, 256)),     # prefill kernel, then a smaller prefill
    ((16, 8192, 200), (9, 2048, 300)),        # unfused decode (rows from global, then staged)
    ((16384, 3072, 1024), (1, 1024, 3072)),   # near the scratch limit, then the fused decode
])
def test_noalloc_matches_forward_two_calls(first, second):
    for seed, (M, K, N) in enumerate((first, second)):
        x, nw, pw, scale = _case(seed + 3 * first[0], M, K, N)
        for norm in (nw, None):
            ref = bl.bitlinear_forward(x, norm, pw, scale, N, EPS)
            y = torch.full((M, N), float("nan"), device=DEV)
            assert _noalloc(x, norm, pw, scale, N, y) == bl.BL_OK
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (M, K, N, norm is None)


def test_noalloc_refuses_sizes_past_the_scratch():
    M, K, N = 32768, 3072, 8  # codes alone are 96 MiB
    x, nw, pw, scale = _case(7, M, K, N)  # full-size buffers: a refusal is the only outcome
    y = torch.empty((M, N), device=DEV)
    st = bl.lib.bitlinear_forward_noalloc(x.data_ptr(), nw.data_ptr(), pw.data_ptr(),
                                          ctypes.c_float(scale), M, K, N, ctypes.c_float(EPS),
                                          y.data_ptr(), None)
    assert st == bl.BL_ERR_UNSUPPORTED
