"""Accuracy of the encoder's Swish (SiLU of the compressor, ResidualKV review page
section 2.3) on the GPU, against fp64.

The kernels evaluate Swish(a) = a / (1 + e^-a) from the hardware 2^x and reciprocal with
a split log2(e), an FMA-recovered product error and one residual correction of the
quotient (kv_cache_compression_residualkv_amd/csrc/rkv_swish.h). The probe library
compiles that same source. This measures its error in units of the last place of the
fp32 result over [-87, 88] (at most 4 ulp, 0.5 ulp on average; about 94 % of the values
are within one ulp, the rest up to 3 ulp, where the hardware 2^x and reciprocal each add
about one ulp), and the absolute error of the clamped tail below -87.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "support", "libswish_probe.so")
MAX_ULP = 4.0


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.rkv_swish_probe.restype = ctypes.c_int
    lib.rkv_swish_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]

    def run(x: np.ndarray) -> np.ndarray:
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        yd = torch.empty_like(xd)
        assert lib.rkv_swish_probe(xd.data_ptr(), yd.data_ptr(), xd.numel(), None) == 0
        torch.cuda.synchronize()
        return yd.cpu().numpy()

    return run


def swish64(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return x / (1.0 + np.exp(-x))


def ulp32(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)


def test_swish_error_in_ulps(probe):
    rng = np.random.default_rng(0)
    grid = np.linspace(-87.0, 88.0, 4_000_001, dtype=np.float32)
    tiny = np.concatenate([2.0 ** np.arange(-126, 1, 0.25), -(2.0 ** np.arange(-126, 1, 0.25))]).astype(np.float32)
    rand = np.concatenate([rng.uniform(-87, 88, 1_000_000), rng.normal(0, 3, 1_000_000)]).astype(np.float32)
    x = np.concatenate([grid, tiny, rand])
    x = x[(x >= -87.0) & (x <= 88.0)]
    y = probe(x).astype(np.float64)
    ref = swish64(x)
    err = np.abs(y - ref) / ulp32(ref)
    worst = int(np.argmax(err))
    print(f"max error {err.max():.3f} ulp at x = {x[worst]!r}; mean {err.mean():.3f} ulp; "
          f"within 1 ulp {np.mean(err <= 1.0):.5f}")
    assert err.max() <= MAX_ULP, (float(err.max()), float(x[worst]))
    assert err.mean() <= 0.5
    assert np.mean(err <= 1.0) >= 0.9


def test_swish_tails(probe):
    # below -87 the argument is clamped: the result stays within 2e-36 of the true value
    lo = np.linspace(-150.0, -87.0, 20001, dtype=np.float32)
    y = probe(lo).astype(np.float64)
    assert np.max(np.abs(y - swish64(lo))) <= 2e-36
    # above 88, e^-a is below the fp32 resolution of 1 + e^-a: Swish(a) = a
    hi = np.linspace(88.0, 1.0e4, 20001, dtype=np.float32)
    assert np.array_equal(probe(hi), hi)
    # Swish(0) = 0 and the sign follows a
    z = probe(np.array([0.0, -0.0, 1e-30, -1e-30], dtype=np.float32))
    assert z[0] == 0.0 and z[1] == 0.0 and z[2] > 0 and z[3] < 0
