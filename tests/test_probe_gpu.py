"""The MFMA-rate probe (measurement support, mfsdp_probe_mfma_bf16) computes
what it claims: with all-one bf16 operands every accumulator element gains
16 per MFMA, 32 per iteration, so each wave's sum is 64 lanes x 256
elements x 32 x iters exactly; with zero operands it is zero."""

import pytest

from matrix_optimizer_owner_amd import binding as B

pytestmark = pytest.mark.gpu


def test_probe_sums_are_exact():
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.full((64 * 4,), -1.0, dtype=torch.float32, device=dev)
    iters = 10
    for fill, want in ((1.0, 64 * 256 * 32 * iters), (0.0, 0.0)):
        ops = torch.full((1 << 16,), fill, dtype=torch.bfloat16, device=dev)
        flops = B.probe_mfma_bf16(ops.data_ptr(), ops.numel() * 2, 64, iters, sink.data_ptr(), stream)
        torch.cuda.synchronize()
        assert flops == 64 * 4 * iters * 32 * 32 * 32 * 16 * 2
        assert bool((sink == want).all()), (fill, sink[:4].tolist())
