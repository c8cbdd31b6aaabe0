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


def test_hbm_probe_copies_and_writes():
    """The streaming probe's copy mode copies, its write mode writes its
    pattern (element i of 16-byte words: i, 0, 0, 0), its read mode leaves
    memory alone."""
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    n = (1 << 20) + 48  # not a multiple of the grid: the bounds of the last pass
    src = torch.randint(0, 2 ** 31 - 1, (n,), dtype=torch.int32, device=dev)
    dst = torch.zeros(n, dtype=torch.int32, device=dev)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)
    B.probe_hbm(dst.data_ptr(), src.data_ptr(), n * 4, 2, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    before = src.clone()
    B.probe_hbm(0, src.data_ptr(), n * 4, 0, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    B.probe_hbm(dst.data_ptr(), 0, n * 4, 1, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    words = dst.view(-1, 4)
    assert torch.equal(words[:, 0], torch.arange(n // 4, dtype=torch.int32, device=dev))
    assert int(words[:, 1:].abs().sum()) == 0
