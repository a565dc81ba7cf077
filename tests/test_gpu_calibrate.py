"""The measurement kernels give exactly what their definitions fix: the XOR of every
32-bit word of the buffer they stream, and 16 * a * b * iters in every accumulator
element of the MFMA loop (bf16 operands, fp32 sums that stay exact below 2^24)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def F():
    import long_context_diffusion_amd as lib
    return lib


@pytest.mark.parametrize("n_words,workgroups", [(4, 1), (16384, 3), (16384 * 5 + 12, 2), (1 << 20, 64)])
def test_calibrate_read_xor(n_words, workgroups):
    print(f"calibrate_read words={n_words} workgroups={workgroups}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(n_words)
    x = torch.randint(-(1 << 31), (1 << 31) - 1, (n_words,), dtype=torch.int32, device="cuda", generator=g)
    sink = F().calibrate_read(x, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(x.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("workgroups,iters,a,b", [(1, 1, 1.0, 1.0), (8, 100, 1.0, 0.5), (256, 1000, -2.0, 0.25)])
def test_calibrate_mfma_value(workgroups, iters, a, b):
    print(f"calibrate_mfma workgroups={workgroups} iters={iters}", flush=True)
    sink = F().calibrate_mfma(workgroups, iters, a, b)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert s.shape == (workgroups * 4, 2)
    assert np.all(s[:, 0] == 16.0 * a * b * iters)
    assert np.all(s[:, 1] == 0.0)
