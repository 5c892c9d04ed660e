"""GPU parity of the block-scaled GEMM against the oracle's dequantize-then-matmul.

The GEMM is fed the oracle's own codes and scales (uploaded in the library layout),
so these tests isolate it from the quantizer.  Tolerance: relative Frobenius
error <= 1e-3 against the oracle's bf16 output and every element within two bf16
steps plus the worst-case fp32 accumulation-order bound."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads
from tests._util import accumulation_bound, assert_gemm_close, canonical_to_layout, oracle_quantize

pytestmark = pytest.mark.gpu
DEV = "cuda"


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


def run_gpu_gemm(px, sx, pw, sw, k, gsf_x, gsf_w, bias=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = nv().nvfp4_gemm(t(px), t(canonical_to_layout(sx, k)), t(pw), t(canonical_to_layout(sw, k)),
                          float(gsf_x), float(gsf_w), None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def random_operands(rng, rows, k, lo=0x20, hi=0x60):
    nib = rng.integers(0, 16, size=(rows, k), dtype=np.uint8)
    s8 = rng.integers(lo, hi, size=(rows, k // 16)).astype(np.uint8)
    return o.pack_codes(nib), s8


@pytest.mark.parametrize("m,n,k", [
    (1, 1, 16), (5, 7, 48), (64, 128, 256), (300, 200, 272), (257, 129, 4112), (256, 128, 128),
    (512, 384, 1024), (33, 1000, 208), (1000, 33, 96),
])
@pytest.mark.parametrize("with_bias", [False, True])
def test_random_codes_ragged(m, n, k, with_bias):
    rng = np.random.default_rng(m * 31 + n * 7 + k)
    px, sx = random_operands(rng, m, k)
    pw, sw = random_operands(rng, n, k)
    gx, gw = np.float32(3.0), np.float32(0.75)
    bias = workloads.draw("normal", (n,), 3, n) if with_bias else None
    got = run_gpu_gemm(px, sx, pw, sw, k, gx, gw, bias)
    alpha = o.alpha_of(gx, gw)
    ref = o.nvfp4_gemm(px, sx, pw, sw, alpha, None if bias is None else bias.float().numpy())
    bound = accumulation_bound(o.dequantize(px, sx), o.dequantize(pw, sw), alpha)
    assert_gemm_close(got, ref, bound)


@pytest.mark.parametrize("m,n,k", [(4136, 4120, 352), (4096, 4096, 1024), (4097, 4353, 4128)])
def test_large_tile_path(m, n, k):
    """Shapes big enough for the software-pipelined 256x256 kernel: ragged M and N
    (clamped rows), a partial last K tile, and a bias."""
    rng = np.random.default_rng(m + n + k)
    px, sx = random_operands(rng, m, k)
    pw, sw = random_operands(rng, n, k)
    bias = workloads.draw("normal", (n,), 4, n)
    got = run_gpu_gemm(px, sx, pw, sw, k, 2.0, 0.5, bias)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(m - 40, m), rng.choice(m, 200)]))
    ref = o.nvfp4_gemm(px[rows], sx[rows], pw, sw, o.alpha_of(2.0, 0.5), bias.float().numpy())
    bound = accumulation_bound(o.dequantize(px[rows], sx[rows]), o.dequantize(pw, sw), o.alpha_of(2.0, 0.5))
    assert_gemm_close(got[rows], ref, bound)


@pytest.mark.parametrize("m,n,k", [(4096, 1024, 5120), (4096, 5120, 1024), (1000, 3000, 640), (4296, 1024, 5120),
                                   (4096, 1024, 8192)])
def test_split_k_tail(m, n, k):
    """Tiles past the last whole round are split along K into a workspace and summed in a
    fixed order: same oracle tolerance, bitwise repeatable, and close to the unsplit run.
    Up to K = 6144 the 256-row tail tiles run as 128-row halves (a ragged last tile row
    in the third and fourth cases); at K = 8192 as whole tiles."""
    rng = np.random.default_rng(m * 3 + n + k)
    px, sx = random_operands(rng, m, k)
    pw, sw = random_operands(rng, n, k)
    bias = workloads.draw("normal", (n,), 5, n)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = (t(px), t(canonical_to_layout(sx, k)), t(pw), t(canonical_to_layout(sw, k)), 2.0, 0.5, bias.to(DEV))
    a = nv().nvfp4_gemm(*args)
    b = nv().nvfp4_gemm(*args)
    c = nv().nvfp4_gemm(*args, split_k=False)
    # a workspace full of garbage: every partial is written before it is read
    ws = torch.full((nv().gemm_workspace_bytes(m, k, n),), 0x7F, dtype=torch.uint8, device=DEV)
    d = nv().nvfp4_gemm(*args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, d)
    got = a.float().cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(m - 8, m), rng.choice(m, 120)]))
    alpha = o.alpha_of(2.0, 0.5)
    ref = o.nvfp4_gemm(px[rows], sx[rows], pw, sw, alpha, bias.float().numpy())
    bound = accumulation_bound(o.dequantize(px[rows], sx[rows]), o.dequantize(pw, sw), alpha)
    assert_gemm_close(got[rows], ref, bound)
    assert_gemm_close(c.float().cpu().numpy()[rows], ref, bound)


def test_full_scale_range():
    # every E4M3 byte including subnormal scales and zero
    rng = np.random.default_rng(9)
    px, sx = random_operands(rng, 96, 512, 0, 127)
    pw, sw = random_operands(rng, 160, 512, 0, 127)
    got = run_gpu_gemm(px, sx, pw, sw, 512, 1.0, 1.0)
    ref = o.nvfp4_gemm(px, sx, pw, sw, np.float32(1.0))
    assert_gemm_close(got, ref, accumulation_bound(o.dequantize(px, sx), o.dequantize(pw, sw), 1.0))


def test_one_hot_products_are_exact():
    # one nonzero code per row: each output is a single exact product
    m, n, k = 64, 96, 384
    nx = np.zeros((m, k), np.uint8)
    nw = np.zeros((n, k), np.uint8)
    rng = np.random.default_rng(4)
    cols = rng.integers(0, k, size=m)
    nx[np.arange(m), cols] = rng.integers(1, 16, size=m)
    nw[np.arange(n), cols[np.arange(n) % m]] = rng.integers(1, 16, size=n)
    sx = rng.integers(0x30, 0x50, size=(m, k // 16)).astype(np.uint8)
    sw = rng.integers(0x30, 0x50, size=(n, k // 16)).astype(np.uint8)
    px, pw = o.pack_codes(nx), o.pack_codes(nw)
    got = run_gpu_gemm(px, sx, pw, sw, k, 1.0, 1.0)
    ref = o.nvfp4_gemm(px, sx, pw, sw, np.float32(1.0))
    assert np.array_equal(got, ref)


def test_tiny_linear_gemm():
    lin = workloads.tiny_linear()
    x = lin.x.float().numpy()
    w = lin.w.float().numpy()
    pw, sw, gw = o.quantize_weight(w)
    r = o.nvfp4_linear_inference(x, pw, sw, gw, lin.bias.float().numpy())
    got = run_gpu_gemm(r["codes"], r["scales"], pw, sw, lin.k, r["gsf_x"], gw, lin.bias)
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(got, r["out"], bound)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gate", "q_proj", "o_proj", "down"])
def test_full_size_sampled_rows(name):
    """Full-size problems through nvfp4_linear (the benchmark's launch), checked on
    64 sampled rows against the oracle, plus the W4A4 probe on those rows."""
    print(f"[full-size gemm] {name}", flush=True)
    if name == "gate":
        lin = workloads.headline_gate()
    elif name == "down":
        lin = workloads.qwen3_mlp(which=("down",))[0]
    else:
        lin = {l.name.split(".")[1]: l for l in workloads.qwen3_attention()}[name]
    x = lin.x.to(DEV)
    w = lin.w.to(DEV)
    packed, inv_scale, gsf_w = nv().quantize_weight(w)
    out = nv().nvfp4_linear(x, packed, inv_scale, gsf_w, None, lin.n)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(lin.m, 64, replace=False))
    xf = lin.x.float().numpy()
    wf = lin.w.float().numpy()
    gx = o.global_sf(o.amax(xf))
    gw = o.global_sf(o.amax(wf))
    pw, sw = oracle_quantize(wf, gw)
    assert np.float32(gsf_w.item()) == gw
    assert np.array_equal(packed.cpu().numpy(), pw)
    px, sx = oracle_quantize(xf[rows], gx)
    alpha = o.alpha_of(gx, gw)
    ref = o.nvfp4_gemm(px, sx, pw, sw, alpha)
    got = out[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    bound = accumulation_bound(o.dequantize(px, sx), o.dequantize(pw, sw), alpha)
    assert_gemm_close(got, ref, bound)
    err = o.probe_relative_error(got, xf[rows], wf)
    print(f"  probe relative error vs bf16 product: {err:.4f}", flush=True)
    assert 0.10 < err < 0.16


def test_probe_near_the_pages_figure():
    """512 random N(0,1) rows through a Qwen3-shaped weight: ||out - xW^T|| / ||xW^T|| ~ 0.13."""
    x = workloads.draw("normal", (512, 5120), 99, 0)
    w = workloads.draw("normal", (1024, 5120), 99, 1, 0.02)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    out = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, None, 1024)
    err = o.probe_relative_error(out.float().cpu().numpy(), x.float().numpy(), w.float().numpy())
    assert abs(err - 0.13) < 0.015, err
    # scales that do not belong to the codes are far off
    bad = inv_scale[torch.randperm(inv_scale.numel(), device=DEV)]
    out_bad = nv().nvfp4_linear(x.to(DEV), packed, bad, gsf_w, None, 1024)
    err_bad = o.probe_relative_error(out_bad.float().cpu().numpy(), x.float().numpy(), w.float().numpy())
    assert err_bad > 2.5 * err


@pytest.mark.parametrize("m", [1, 5, 16, 17, 40, 64, 100, 128])
@pytest.mark.parametrize("n,k", [(1024, 5120), (300, 4128), (5120, 1024), (301, 1056)])
def test_few_rows_weight_streaming(m, n, k):
    """Decode shapes (M <= 128): the weight-streaming kernels (up to 32 rows, 64 on narrow
    weights) and the pipelined one above, with and without their K splits, against the
    oracle; ragged and odd N and a partial last K tile."""
    rng = np.random.default_rng(m * 7 + n + k)
    px, sx = random_operands(rng, m, k)
    pw, sw = random_operands(rng, n, k)
    bias = workloads.draw("normal", (n,), 6, n)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = (t(px), t(canonical_to_layout(sx, k)), t(pw), t(canonical_to_layout(sw, k)), 1.5, 0.25, bias.to(DEV))
    split = nv().nvfp4_gemm(*args)
    again = nv().nvfp4_gemm(*args)
    whole = nv().nvfp4_gemm(*args, split_k=False)
    torch.cuda.synchronize()
    assert torch.equal(split, again)
    alpha = o.alpha_of(1.5, 0.25)
    ref = o.nvfp4_gemm(px, sx, pw, sw, alpha, bias.float().numpy())
    bound = accumulation_bound(o.dequantize(px, sx), o.dequantize(pw, sw), alpha)
    assert_gemm_close(split.float().cpu().numpy(), ref, bound)
    assert_gemm_close(whole.float().cpu().numpy(), ref, bound)


@pytest.mark.parametrize("n,k,split_k", [(1024, 5120, True), (5120, 8192, True), (4096, 5120, True),
                                         (300, 4128, True), (301, 1056, True), (64, 96, True), (200, 25600, True),
                                         (64, 16384, False)])
def test_one_row_decode_equals_row_of_two(n, k, split_k):
    """Decode rows are independent: one activation row gives the first row of the same
    product with a second row added, bit for bit, and is within the oracle's bound.
    Shapes: 8-wave blocks (k, o), 4-wave blocks, a partial last super tile, a single K
    tile, a 12-way K split, and unsplit 16384-long rows on 8-wave blocks."""
    rng = np.random.default_rng(n + 3 * k)
    px, sx = random_operands(rng, 2, k)
    pw, sw = random_operands(rng, n, k)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    w = (t(pw), t(canonical_to_layout(sw, k)))
    two = nv().nvfp4_gemm(t(px), t(canonical_to_layout(sx, k)), *w, 1.5, 0.25, split_k=split_k)
    one = nv().nvfp4_gemm(t(px[:1]), t(canonical_to_layout(sx[:1], k)), *w, 1.5, 0.25, split_k=split_k)
    torch.cuda.synchronize()
    assert torch.equal(one[0], two[0])
    alpha = o.alpha_of(1.5, 0.25)
    ref = o.nvfp4_gemm(px[:1], sx[:1], pw, sw, alpha)
    bound = accumulation_bound(o.dequantize(px[:1], sx[:1]), o.dequantize(pw, sw), alpha)
    assert_gemm_close(one.float().cpu().numpy(), ref, bound)


@pytest.mark.parametrize("m,n,k", [(65, 4352, 1056), (200, 4100, 2080), (511, 1000, 640), (128, 25600, 512),
                                   (100, 65800, 256)])
def test_mid_rows_pipelined_split(m, n, k):
    """Between the decode and the full-tile shapes: the pipelined kernel on ragged
    128x256 (M <= 128) or 256x256 tiles, split along K up to one tile per compute
    unit; the last case fills a whole round of 128-row tiles and leaves two more."""
    rng = np.random.default_rng(m + 3 * n + k)
    px, sx = random_operands(rng, m, k)
    pw, sw = random_operands(rng, n, k)
    bias = workloads.draw("normal", (n,), 7, n)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = (t(px), t(canonical_to_layout(sx, k)), t(pw), t(canonical_to_layout(sw, k)), 0.5, 3.0, bias.to(DEV))
    a = nv().nvfp4_gemm(*args)
    b = nv().nvfp4_gemm(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    cols = np.unique(np.concatenate([np.arange(n - 20, n), rng.choice(n, 400)]))
    alpha = o.alpha_of(0.5, 3.0)
    ref = o.nvfp4_gemm(px, sx, pw[cols], sw[cols], alpha, bias.float().numpy()[cols])
    bound = accumulation_bound(o.dequantize(px, sx), o.dequantize(pw[cols], sw[cols]), alpha)
    assert_gemm_close(a.float().cpu().numpy()[:, cols], ref, bound)
