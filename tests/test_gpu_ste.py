"""The straight-through training path (nvfp4_linear_train) on the GPU.

Forward: bit-identical to the inference nvfp4_linear on the packed master weight.
Backward: the gradients of the full-precision linear (quantization as the identity,
chained through the block rotation), checked against the oracle's float64 gradients."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


def _close(got, ref, rel_fro, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= rel_fro, f"{what}: relative Frobenius error {rel:.3e} > {rel_fro}"
    # each element within one part in 2^7 (bf16 outputs round at 2^-9) plus 1e-3 of the rms
    tol = 2.0 ** -7 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, first at {tuple(np.argwhere(bad)[0])}"


@pytest.mark.parametrize("g", [0, 16])
@pytest.mark.parametrize("bias", [False, True])
def test_ste_forward_and_backward(g, bias):
    m, n, k = 96, 320, 1024
    x0 = workloads.draw("t3", (m, k), 21, g)
    w0 = workloads.draw("normal", (n, k), 21, 100 + g, 0.02).float()
    b0 = workloads.draw("normal", (n,), 21, 200, 0.01).float() if bias else None
    gy0 = workloads.draw("normal", (m, n), 21, 300 + g)
    w_master = o.fold_weight(w0.numpy(), g) if g else w0.numpy()          # the rotated master, fp32 values
    x = x0.to(DEV).requires_grad_(True)
    w = torch.from_numpy(np.ascontiguousarray(w_master, dtype=np.float32)).to(DEV).requires_grad_(True)
    b = b0.to(DEV).requires_grad_(True) if bias else None
    y = nv().nvfp4_linear_train(x, w, b, None, g)
    # forward: the inference linear on the packed master weight
    packed, inv_scale, gsf_w = nv().quantize_weight(w.detach().to(torch.bfloat16))
    ref_y = nv().nvfp4_linear(x.detach(), packed, inv_scale, gsf_w,
                              None if b is None else b.detach().to(torch.bfloat16), n, None, g)
    assert torch.equal(y.detach(), ref_y)
    y.backward(gy0.to(DEV))
    torch.cuda.synchronize()
    r = o.ste_linear_grads(gy0.float().numpy(), x0.float().numpy(), w_master, g, with_bias=bias)
    assert x.grad.dtype == torch.bfloat16 and w.grad.dtype == torch.float32
    _close(x.grad.float().cpu().numpy(), r["grad_x"], 5e-3, "grad_x")
    _close(w.grad.cpu().numpy(), r["grad_w"], 1e-4, "grad_w")
    if bias:
        _close(b.grad.cpu().numpy(), r["grad_b"], 1e-5, "grad_b")
