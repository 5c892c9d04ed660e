"""nvfp4_linear_noalloc: the allocation-free entry point against nvfp4_linear.

The no-alloc call runs nvfp4_linear's kernels on the library's fixed device scratch.
Where the whole nvfp4_linear workspace fits in that scratch the two results are
bit-identical; where only the unsplit layout fits, the GEMM's last round of tiles runs
unsplit and the results agree to the GEMM tolerance (and both match the oracle).
Every call goes through the C ABI (the binding only marshals arguments).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as o
import workloads
from tests._util import accumulation_bound, assert_gemm_close

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


def _case(m, k, n, seed, bias=True):
    x = workloads.draw("normal", (m, k), seed, 0)
    w = workloads.draw("normal", (n, k), seed, 1, 0.02)
    b = workloads.draw("normal", (n,), seed, 2, 0.01) if bias else None
    return x, w, b


def _oracle_rows(x, w, b, rows, g=0, gsf_x=None):
    xf = x.float().numpy()
    wf = o.fold_weight(w.float().numpy(), g) if g else w.float().numpy()
    pw, sw, gw = o.quantize_weight(wf)
    if g:
        xf = o.rotate_activation(xf, g)
    gx = o.global_sf(o.amax(xf)) if gsf_x is None else np.float32(gsf_x)
    nib, s8 = o.nvfp4_quantize(xf[rows], gx)
    alpha = o.alpha_of(gx, gw)
    ref = o.nvfp4_gemm(o.pack_codes(nib), s8, pw, sw, alpha, None if b is None else b.float().numpy())
    bound = accumulation_bound(o.dequantize(o.pack_codes(nib), s8), o.dequantize(pw, sw), alpha)
    return ref, bound


def _run_pair(x, w, b, g=0, gsf_x=None):
    lib = nv()
    wd = w.to(DEV)
    if g:
        wd = lib.rotate_activation(wd.float(), g, out_dtype=torch.bfloat16)
    packed, inv_scale, gsf_w = lib.quantize_weight(wd)
    xd = x.to(DEV)
    bd = None if b is None else b.to(DEV)
    gx = None if gsf_x is None else torch.tensor(gsf_x, dtype=torch.float32, device=DEV)
    n = w.shape[0]
    ref = lib.nvfp4_linear(xd, packed, inv_scale, gsf_w, bd, n, gx, g)
    out = torch.full_like(ref, float("nan"))
    got = lib.nvfp4_linear_noalloc(xd, packed, inv_scale, gsf_w, bd, n, gx, g, out=out)
    torch.cuda.synchronize()
    return got, ref


def test_two_calls_in_a_row_second_smaller():
    # call 1: 2048 x 5120 -> 3072 with bias, dynamic scale (pipelined GEMM with a
    # split-K tail, whole workspace in the scratch): bit-identical to nvfp4_linear
    x, w, b = _case(2048, 5120, 3072, 41)
    print("no-alloc call 1: [2048, 5120] x [3072, 5120], dynamic scale, bias", flush=True)
    got, ref = _run_pair(x, w, b)
    assert torch.equal(got, ref)
    rows = np.arange(0, 2048, 97)
    r, bound = _oracle_rows(x, w, b, rows)
    assert_gemm_close(got[torch.from_numpy(rows).to(DEV)].float().cpu().numpy(), r, bound)
    # call 2, smaller: 37 x 1024 -> 300, static scale, on the scratch the first call left
    x, w, b = _case(37, 1024, 300, 42)
    print("no-alloc call 2: [37, 1024] x [300, 1024], static scale, bias", flush=True)
    got, ref = _run_pair(x, w, b, gsf_x=20.0)
    assert torch.equal(got, ref)
    r, bound = _oracle_rows(x, w, b, np.arange(37), gsf_x=20.0)
    assert_gemm_close(got.float().cpu().numpy(), r, bound)


def test_decode_rows_with_rotation():
    # 3 rows (the fp16-activation decode path), group-16 rotation, dynamic scale
    x, w, b = _case(3, 4096, 1024, 43, bias=False)
    print("no-alloc: [3, 4096] x [1024, 4096], rotation 16", flush=True)
    got, ref = _run_pair(x, w, b, g=16)
    assert torch.equal(got, ref)
    r, bound = _oracle_rows(x, w, b, np.arange(3), g=16)
    assert_gemm_close(got.float().cpu().numpy(), r, bound)


def test_one_row_single_launch():
    # one row (the decode GEMM quantizes the row itself), dynamic then static scale; the
    # dynamic scale lands in the scratch for the epilogue and the split-K reduce
    x, w, b = _case(1, 5120, 1024, 45)
    for gsf_x in (None, 30.0):
        print(f"no-alloc: [1, 5120] x [1024, 5120], scale {gsf_x}", flush=True)
        got, ref = _run_pair(x, w, b, gsf_x=gsf_x)
        assert torch.equal(got, ref)
        r, bound = _oracle_rows(x, w, b, np.arange(1), gsf_x=gsf_x)
        assert_gemm_close(got.float().cpu().numpy(), r, bound)


@pytest.mark.slow
def test_unsplit_when_only_the_codes_fit():
    # down_proj shape: the split-K partials (67 MB) do not fit beside the codes, so the
    # no-alloc call runs the tail unsplit: same function, summation order aside
    m, k, n = 4096, 25600, 5120
    x, w, _ = _case(m, k, n, 44, bias=False)
    print(f"no-alloc: [{m}, {k}] x [{n}, {k}], unsplit tail", flush=True)
    got, ref = _run_pair(x, w, None)
    rows = np.arange(5, m, 509)
    sel = torch.from_numpy(rows).to(DEV)
    r, bound = _oracle_rows(x, w, None, rows)
    assert_gemm_close(got[sel].float().cpu().numpy(), r, bound)
    assert_gemm_close(ref[sel].float().cpu().numpy(), r, bound)
    diff = torch.linalg.vector_norm((got.float() - ref.float()).flatten())
    assert float(diff) <= 1e-3 * float(torch.linalg.vector_norm(ref.float().flatten()))


def test_too_large_is_rejected_before_any_work():
    lib = nv()
    L = lib._lib.lib()
    fake = ctypes.c_void_p(0x1000)
    rc = L.nvfp4_linear_noalloc(fake, 16384, 16384, fake, fake, fake, None, 1024, None, 0, fake, None)
    assert rc == lib._lib.NVFP4_ERR_WORKSPACE
    assert "fixed" in L.nvfp4_last_error().decode()
