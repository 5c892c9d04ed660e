"""GPU parity of the amax / global-scale, rotation and quantize kernels against the
CPU oracle: every code byte, scale byte and global scale must be identical."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads
from tests._util import canonical_to_layout, layout_padding, layout_to_canonical, oracle_quantize

pytestmark = pytest.mark.gpu
DEV = "cuda"


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


def gpu_quantize(x_cpu: torch.Tensor, gsf=None, g: int = 0):
    x = x_cpu.to(DEV)
    m, k = x.shape
    codes, scales, used = nv().quantize_activation(x, gsf, g)
    torch.cuda.synchronize()
    lay = scales.cpu().numpy()
    assert not layout_padding(lay, m, k).any(), "scale padding bytes must be zero"
    return codes.cpu().numpy(), layout_to_canonical(lay, m, k), np.float32(used.item())


def oracle_expected(x_cpu: torch.Tensor, gsf=None, g: int = 0):
    xf = x_cpu.float().numpy()
    if g:
        xf = o.rotate_activation(xf, g)
    gs = o.global_sf(o.amax(xf)) if gsf is None else np.float32(gsf)
    packed, s8 = oracle_quantize(xf, gs)
    return packed, s8, gs


def assert_same(got, exp, what):
    gc, gs, gg = got
    ec, es, eg = exp
    assert gg.view(np.uint32) == np.float32(eg).view(np.uint32), f"{what}: global scale {gg!r} != {eg!r}"
    assert np.array_equal(gs, es), f"{what}: {int((gs != es).sum())} scale bytes differ"
    assert np.array_equal(gc, ec), f"{what}: {int((gc != ec).sum())} code bytes differ"


def test_tiny_dynamic():
    x = workloads.tiny_linear().x
    assert_same(gpu_quantize(x), oracle_expected(x), "tiny")


@pytest.mark.parametrize("m,k", [(1, 16), (3, 208), (37, 272), (130, 400), (65, 128), (2, 4112), (513, 96)])
@pytest.mark.parametrize("static", [False, True])
def test_ragged_shapes(m, k, static):
    x = workloads.draw("t3", (m, k), 21, m * 7 + k)
    gsf = 3.5 if static else None
    assert_same(gpu_quantize(x, gsf), oracle_expected(x, gsf), f"{m}x{k}")


def test_zero_input():
    x = torch.zeros((5, 64), dtype=torch.bfloat16)
    got = gpu_quantize(x)
    assert_same(got, oracle_expected(x), "zeros")
    assert not got[0].any() and not got[1].any()


def test_exhaustive_sweep_unit_scale():
    """Unit global scale: for every nonzero E4M3 level s a block whose max is exactly
    6*s forces scale byte s; its other 15 slots sweep every bf16 value with |v| <= 6s."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    rows = []
    for s8 in range(1, 127):
        top = np.float32(6.0 * o.E4M3_VALUES[s8])
        cand = vals[np.abs(vals) <= top]
        nfill = (-len(cand)) % 15
        cand = np.concatenate([cand, np.zeros(nfill, np.float32)]).reshape(-1, 15)
        blocks = np.concatenate([np.full((cand.shape[0], 1), top, np.float32), cand], axis=1)
        rows.append(blocks)
    blocks = np.concatenate(rows)
    pad = (-blocks.shape[0]) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 16), np.float32)])
    x = torch.from_numpy(blocks.reshape(-1, 128)).to(torch.bfloat16)   # 8 blocks per row
    assert np.array_equal(x.float().numpy().reshape(-1, 16), blocks)   # all exact in bf16
    got = gpu_quantize(x, 1.0)
    exp = oracle_expected(x, 1.0)
    assert_same(got, exp, "sweep")
    # every level appears as the scale of its own blocks
    assert set(np.unique(exp[1])) >= set(range(1, 127))


def test_weight_quantizer_matches_oracle():
    for w_cpu in (workloads.tiny_linear().w, workloads.draw("normal", (1024, 5120), 1, 12, 0.02)):
        w = w_cpu.to(DEV)
        packed, scales, gsf = nv().quantize_weight(w)
        torch.cuda.synchronize()
        pw, sw, gw = o.quantize_weight(w_cpu.float().numpy())
        n, k = w_cpu.shape
        assert np.float32(gsf.item()) == gw
        assert np.array_equal(layout_to_canonical(scales.cpu().numpy(), n, k), sw)
        assert np.array_equal(packed.cpu().numpy(), pw)


@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128])
def test_rotation_bitwise(g):
    x = workloads.draw("t3", (33, 512), 5, g)
    y = nv().rotate_activation(x.to(DEV), g)
    ref = o.rotate_activation(x.float().numpy(), g)
    assert np.array_equal(y.float().cpu().numpy().view(np.uint32), ref.view(np.uint32))
    # the fp32 weight fold: f32 -> f32 and f32 -> bf16
    wf = workloads.draw("normal", (40, 256), 6, g, 0.02).float()
    y32 = nv().rotate_activation(wf.to(DEV), g)
    ref32 = o.rotate_activation(wf.numpy(), g, out="f32")
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
    yb = nv().rotate_activation(wf.to(DEV), g, out_dtype=torch.bfloat16)
    assert np.array_equal(yb.float().cpu().numpy(), o.fold_weight(wf.numpy(), g))


@pytest.mark.parametrize("g", [2, 16, 128])
def test_fused_rotation_equals_rotate_then_quantize(g):
    x = workloads.draw("t3", (300, 1024), 8, g).to(DEV)
    fused = nv().quantize_activation(x, None, g)
    xr = nv().rotate_activation(x, g)
    split = nv().quantize_activation(xr, None, 0)
    for a, b in zip(fused, split):
        assert torch.equal(a, b)
    assert_same(gpu_quantize(x.cpu(), None, g), oracle_expected(x.cpu(), None, g), f"rot{g}")


@pytest.mark.parametrize("m,k,g", [(4096, 5120, 0), (4096, 5248, 0), (4096, 4096, 16), (4096, 4224, 16),
                                   (1, 16, 0), (37, 272, 0), (37, 272, 16), (300, 1024, 2), (513, 4224, 128)])
def test_dynamic_equals_static_at_its_amax(m, k, g):
    """The dynamic quantize (amax pass, then the quantize pass taking the max of the
    partials) writes the same codes, scales and global scale as the static-scale pass
    given the scale that the calibration kernels (nvfp4_amax, then
    nvfp4_static_global_scale at margin 1) form from x: two kernel sequences that share
    only the per-block encoder."""
    print(f"[dynamic vs static quantize] {m}x{k} rot{g}", flush=True)
    x = workloads.draw("t3", (m, k), 31, m + k + g).to(DEV)
    gsf = nv().static_global_sf(nv().amax(x, g), 1.0)
    dc, ds, dg = nv().quantize_activation(x, None, g)
    sc, ss, sg = nv().quantize_activation(x, gsf, g)
    torch.cuda.synchronize()
    assert dg.item() == gsf.item() == sg.item()
    assert torch.equal(ds, ss), f"{int((ds != ss).sum())} scale bytes differ"
    assert torch.equal(dc, sc), f"{int((dc != sc).sum())} code bytes differ"
    # and twice in a row: nothing carries over from one call to the next
    dc2, ds2, dg2 = nv().quantize_activation(x, None, g)
    torch.cuda.synchronize()
    assert torch.equal(dc2, dc) and torch.equal(ds2, ds) and dg2.item() == dg.item()


FULL = [
    ("qwen3 attention x [4096,5120]", lambda: workloads.qwen3_attention()[0].x, 0),
    ("qwen3 o_proj x [4096,8192]", lambda: workloads.qwen3_attention()[3].x, 0),
    ("qwen3 down_proj x silu(g)*u [4096,25600]", lambda: workloads.qwen3_mlp(which=("down",))[0].x, 0),
    ("vit tile fc_out x t3 [4096,4096] rot16", lambda: workloads.vit_decoder_tiles(tiles=1, which=("fc_out",))[0].x, 16),
    ("vit tile qkv x t3 [4096,1024] rot16", lambda: workloads.vit_decoder_tiles(tiles=1, which=("qkv",))[0].x, 16),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,make,g", FULL, ids=[f[0].split(" x")[0].replace(" ", "_") for f in FULL])
def test_full_size_bitwise(name, make, g):
    print(f"[full-size quantize] {name}", flush=True)
    x = make()
    assert_same(gpu_quantize(x, None, g), oracle_expected(x, None, g), name)


@pytest.mark.parametrize("m", [1, 16, 128])
def test_small_m_bitwise(m):
    for lin in workloads.small_m_sweep(ms=(m,)):
        if lin.name.endswith(("k_proj", "up_proj")):     # same K as v/gate; keep the sweep short
            continue
        assert_same(gpu_quantize(lin.x), oracle_expected(lin.x), lin.name)


@pytest.mark.parametrize("rows,k", [(1, 16), (37, 272), (300, 1024), (5, 4112)])
@pytest.mark.parametrize("gsf", [1.0, 8.0, 2688.0 / 3.7, 1.0e-3])
def test_dequantize_bitwise(rows, k, gsf):
    """NVFP4 -> bf16 / fp32 expansion bit-exact against the oracle over every E4M3 byte
    (subnormal and zero scales included) and signed zero codes."""
    rng = np.random.default_rng(rows + k)
    nib = rng.integers(0, 16, size=(rows, k), dtype=np.uint8)
    s8 = rng.integers(0, 127, size=(rows, k // 16)).astype(np.uint8)
    packed = o.pack_codes(nib)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    lay = t(canonical_to_layout(s8, k))
    g = np.float32(gsf)
    for dtype, mode in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        got = nv().dequantize(t(packed), lay, float(g), dtype)
        ref = o.dequantize_values(packed, s8, g, out=mode)
        if dtype == torch.bfloat16:
            assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), o.f32_to_bf16_bits(ref))
        else:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dequantized_weight_of_a_layer():
    lin = workloads.tiny_linear()
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV))
    pw, sw, gw = o.quantize_weight(lin.w.float().numpy())
    got = layer.dequantized_weight().float().cpu().numpy()
    assert np.array_equal(got, o.dequantize_values(pw, sw, gw))


@pytest.mark.parametrize("m,k,g", [(32, 4096, 0), (33, 4096, 0), (1, 131072, 16), (2, 65536, 128), (8, 16400, 0),
                                   (8192, 16, 0), (1, 5120, 0), (3, 25600, 16), (16, 5120, 0), (24, 5120, 16),
                                   (12, 5120, 0), (25, 5120, 0), (5, 48, 2), (2048, 64, 32)])
def test_single_launch_small_dynamic_quantize(m, k, g):
    """Dynamic scale on inputs of at most 2^17 values takes the single-launch quantizer
    (every workgroup takes the abs-max of the whole input itself, then quantizes its
    share; up to 16 workgroups); larger ones the two passes.  Both sides of the
    threshold, one and several workgroups, are bit-exact against the oracle, with and
    without rotation."""
    x = workloads.draw("t3", (m, k), m + k + g, 5)
    assert_same(gpu_quantize(x, None, g), oracle_expected(x, None, g), f"{m}x{k} g{g}")
