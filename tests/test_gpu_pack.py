"""uno_pack_weight against the layout include/uno.h states: element (n, k) of a
row-major [n_out, n_in] matrix goes to ((n/16)*(n_in/32) + k/32)*512 +
((k%32)/8)*128 + (n%16)*8 + k%8 (the weight layout every GEMM reads)."""
import numpy as np
import pytest
import torch

from gpu_util import gpu_or_fail

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_out,n_in", [(16, 32), (48, 96), (512, 4096), (6144, 4096)])
def test_pack_weight_layout(n_out, n_in):
    U = gpu_or_fail()
    rng = np.random.default_rng([n_out, n_in])
    w = rng.integers(0, 1 << 16, size=(n_out, n_in), dtype=np.uint16)
    got = U.pack_weight(torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16))
    torch.cuda.synchronize()
    got = got.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    n = np.arange(n_out)[:, None]
    k = np.arange(n_in)[None, :]
    pos = ((n // 16) * (n_in // 32) + k // 32) * 512 + ((k % 32) // 8) * 128 + (n % 16) * 8 + k % 8
    want = np.empty(n_out * n_in, dtype=np.uint16)
    want[pos.reshape(-1)] = w.reshape(-1)
    np.testing.assert_array_equal(got, want)
