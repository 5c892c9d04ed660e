"""The SwiGLU product feeding down_proj, formed inside the quantizer: bit-exact against
the oracle, and the fused quantizer / linear bit-identical to the unfused two-step path."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads
from tests._util import accumulation_bound, assert_gemm_close, layout_to_canonical

pytestmark = pytest.mark.gpu
DEV = "cuda"


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


def _gate_up(m, k, seed):
    g = workloads.draw("normal", (m, k), seed, 0, 3.0)
    u = workloads.draw("normal", (m, k), seed, 1, 3.0)
    # extremes: clamped exponent range, zeros of both signs, huge and tiny magnitudes
    special = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 79.5, -79.5, 85.0, -85.0, 200.0, -200.0, 1.0, -1.0,
                            1e30, -1e30, 0.5, -0.5], dtype=torch.float32).to(torch.bfloat16)
    g.view(-1)[:16] = special
    if u.numel() >= 32:
        u.view(-1)[16:32] = special
    return g, u


def _bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("m,k", [(1, 16), (37, 272), (3, 25600)])
def test_swiglu_bitwise(m, k):
    g, u = _gate_up(m, k, m + k)
    got = nv().swiglu(g.to(DEV), u.to(DEV))
    ref = o.swiglu_product(g.float().numpy(), u.float().numpy())
    assert np.array_equal(_bf16_bits(got), o.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("m,k", [(37, 272), (130, 2048)])
def test_quantize_swiglu_equals_two_steps_and_oracle(m, k, static):
    g, u = _gate_up(m, k, 3 * m + k)
    gd, ud = g.to(DEV), u.to(DEV)
    gsf = 7.25 if static else None
    c1, s1, f1 = nv().quantize_swiglu(gd, ud, gsf)
    c2, s2, f2 = nv().quantize_activation(nv().swiglu(gd, ud), gsf)
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and f1.item() == f2.item()
    x = o.swiglu_product(g.float().numpy(), u.float().numpy())
    gx = np.float32(gsf) if static else o.global_sf(o.amax(x))
    nib, s8 = o.nvfp4_quantize(x, gx)
    assert np.float32(f1.item()) == gx
    assert np.array_equal(c1.cpu().numpy(), o.pack_codes(nib))
    assert np.array_equal(layout_to_canonical(s1.cpu().numpy(), m, k), s8)


@pytest.mark.parametrize("m,n", [(5, 640), (256, 640)])
def test_linear_swiglu(m, n):
    """down_proj-shaped (K = 25600): the fused call equals the unfused one bit for bit,
    and both match the oracle."""
    k = 25600
    g, u = workloads.down_proj_gate_up(m=m, k=k)
    w = workloads.draw("normal", (n, k), 21, n, 0.02)
    bias = workloads.draw("normal", (n,), 22, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    gd, ud = g.to(DEV), u.to(DEV)
    fused = nv().nvfp4_linear_swiglu(gd, ud, packed, inv_scale, gsf_w, bias.to(DEV), n)
    two = nv().nvfp4_linear(nv().swiglu(gd, ud), packed, inv_scale, gsf_w, bias.to(DEV), n)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    x = o.swiglu_product(g.float().numpy(), u.float().numpy())
    pw, sw, gw = o.quantize_weight(w.float().numpy())
    r = o.nvfp4_linear_inference(x, pw, sw, gw, bias.float().numpy())
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(fused.float().cpu().numpy(), r["out"], bound)


@pytest.mark.slow
def test_full_size_down_proj_fused():
    """The full down_proj (x from gate/up [4096, 25600], W [5120, 25600]) through the fused
    call: equal to the two-step path everywhere, and to the oracle on 48 sampled rows."""
    print("[full-size fused down_proj]", flush=True)
    m, k, n = 4096, 25600, 5120
    g, u = workloads.down_proj_gate_up(m=m, k=k)
    w = workloads.small_m_weight("mlp.down_proj")          # the Qwen3-shaped down_proj weight
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    gd, ud = g.to(DEV), u.to(DEV)
    fused = nv().nvfp4_linear_swiglu(gd, ud, packed, inv_scale, gsf_w, None, n)
    two = nv().nvfp4_linear(nv().swiglu(gd, ud), packed, inv_scale, gsf_w, None, n)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    x = o.swiglu_product(g.float().numpy(), u.float().numpy())
    gx = o.global_sf(o.amax(x))
    rows = np.sort(np.random.default_rng(1).choice(m, 48, replace=False))
    nib, s8 = o.nvfp4_quantize(x[rows], gx)
    wf = w.float().numpy()
    gw = o.global_sf(o.amax(wf))
    from tests._util import oracle_quantize
    pw, sw = oracle_quantize(wf, gw)
    alpha = o.alpha_of(gx, gw)
    ref = o.nvfp4_gemm(o.pack_codes(nib), s8, pw, sw, alpha)
    bound = accumulation_bound(o.dequantize(o.pack_codes(nib), s8), o.dequantize(pw, sw), alpha)
    assert_gemm_close(fused[torch.from_numpy(rows).to(DEV)].float().cpu().numpy(), ref, bound)
