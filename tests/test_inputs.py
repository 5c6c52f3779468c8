"""CPU checks of the seeded input generator (no method arithmetic in it)."""
import torch

from gated_mlp_gemm_amd import inputs


def test_mlp_inputs_extend_the_swiglu_inputs():
    for M, K, N, seed in [(5, 16, 24, 3), (128, 896, 64, 0)]:
        a = inputs.make_inputs(M, K, N, seed)
        b = inputs.make_mlp_inputs(M, K, N, seed)
        assert all(torch.equal(x, y) for x, y in zip(a, b[:3]))
        W3 = b[3]
        assert W3.shape == (N, K) and W3.dtype == torch.bfloat16
        # N(0, 1/N): the sample standard deviation is close to 1/sqrt(N)
        assert abs(float(W3.float().std()) * N ** 0.5 - 1.0) < 0.1
