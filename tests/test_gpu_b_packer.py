"""GPU packer == oracle preshuffle, bit-exact, and unshuffle inverts it."""
import numpy as np
import pytest
import torch

import dense_gemm_packer_amd as dgp
import oracle
import synth
from gpu_common import DEV, dev_codes

pytestmark = pytest.mark.gpu


def _codes(N, K, dtype, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    if dtype == "bf16":
        return g.integers(0, 65536, size=(N, K), dtype=np.uint16)
    return g.integers(0, 256, size=(N, K), dtype=np.uint8)   # every e4m3 code, NaNs included


def _host(t, dtype):
    return t.view(torch.int16 if dtype == "bf16" else torch.uint8).cpu().numpy().view(
        np.uint16 if dtype == "bf16" else np.uint8)


@pytest.mark.parametrize("dtype,N,K", [("bf16", 16, 32), ("bf16", 48, 96), ("bf16", 256, 256),
                                       ("fp8", 16, 64), ("fp8", 32, 448), ("fp8", 2048, 7168),
                                       ("bf16", 512, 8192)])
def test_packer_matches_oracle_bit_exact(dtype, N, K):
    B = _codes(N, K, dtype, N + K)
    Bs = dgp.preshuffle_b(dev_codes(B, dtype))
    torch.cuda.synchronize()
    want = oracle.preshuffle_b(B)
    assert np.array_equal(_host(Bs, dtype), want)
    back = dgp.unshuffle_b(Bs)
    torch.cuda.synchronize()
    assert np.array_equal(_host(back, dtype), B)


def test_packer_full_size_weights():
    """The weights of the 4096x8192 bf16 workload and the 16384x7168 fp8
    decode workload, bit-exact against the oracle."""
    w = synth.workload_inputs("bf16_large", M=16)
    Bs = dgp.preshuffle_b(dev_codes(w["B"], "bf16"))
    torch.cuda.synchronize()
    assert np.array_equal(_host(Bs, "bf16"), oracle.preshuffle_b(w["B"]))
    w = synth.workload_inputs("fp8_decode", M=1, N=16384)
    Bs = dgp.preshuffle_b(dev_codes(w["B"], "fp8"))
    torch.cuda.synchronize()
    assert np.array_equal(_host(Bs, "fp8"), oracle.preshuffle_b(w["B"]))


def test_packer_rejects_through_binding():
    with pytest.raises(dgp.DgpError):
        dgp.preshuffle_b(torch.zeros((24, 64), dtype=torch.bfloat16, device=DEV))
