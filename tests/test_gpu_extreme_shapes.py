"""nvfp4_linear at extreme shapes against the oracle: a very tall input (65536 rows, the
quantize grid loops and 256 tile rows), a very long K (131072: the decode kernel's
deepest K split and the two-pass dynamic quantize over a million values) and a very wide
weight (1048576 outputs: 65536 decode tiles), and one row at the last two (the single
launch that quantizes the row inside the decode GEMM).  Index arithmetic that overflows 32 bits
or a grid that covers too little fails here.  Codes and scales of the activation are
bit-exact against the oracle; outputs on sampled rows and columns are within the GEMM
tolerance."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads
from tests._util import accumulation_bound, assert_gemm_close, layout_to_canonical

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


@pytest.mark.parametrize("m,k,n", [(65536, 256, 64), (8, 131072, 64), (4, 64, 1 << 20), (1, 131072, 64), (1, 64, 1 << 20)])
def test_extreme_shape(m, k, n):
    print(f"[extreme shape] m={m} k={k} n={n}", flush=True)
    x = workloads.draw("t3", (m, k), 61, m, 1.0)
    w = workloads.draw("normal", (n, k), 62, n, 0.02)
    bias = workloads.draw("normal", (n,), 63, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    out = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, bias.to(DEV), n)
    codes, scales, gsf = nv().quantize_activation(x.to(DEV))
    torch.cuda.synchronize()
    xf = x.float().numpy()
    gx = o.global_sf(o.amax(xf))
    assert np.float32(gsf.item()) == gx
    nib, s8 = o.nvfp4_quantize(xf, gx)
    assert np.array_equal(codes.cpu().numpy(), o.pack_codes(nib))
    assert np.array_equal(layout_to_canonical(scales.cpu().numpy(), m, k), s8)
    rng = np.random.default_rng(m + k + n)
    rows = np.unique(np.concatenate([rng.choice(m, min(m, 64), replace=False), [m - 1]]))
    cols = np.unique(np.concatenate([rng.choice(n, min(n, 64), replace=False), [n - 1]]))
    wf = w.float().numpy()[cols]
    gw = o.global_sf(o.amax(w.float().numpy()))
    assert np.float32(gsf_w.item()) == gw
    nw, sw = o.nvfp4_quantize(wf, gw)
    pw = o.pack_codes(nw)
    assert np.array_equal(packed[torch.from_numpy(cols).to(DEV)].cpu().numpy(), pw)
    px = o.pack_codes(nib[rows])
    ref = o.nvfp4_gemm(px, s8[rows], pw, sw, o.alpha_of(gx, gw), bias.float().numpy()[cols])
    bound = accumulation_bound(o.dequantize(px, s8[rows]), o.dequantize(pw, sw), o.alpha_of(gx, gw))
    got = out[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]
    assert_gemm_close(got.float().cpu().numpy(), ref, bound)
