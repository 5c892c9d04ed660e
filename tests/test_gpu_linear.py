"""End-to-end nvfp4_linear on the GPU against the oracle, the fusion and per-tile
contracts, activation-scale modes, and error handling through the binding."""
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


def check_against_oracle(lin, x_cpu, out_gpu, packed, inv_scale, gsf_w, global_sf_x=None, g=0, bias=None):
    xf = x_cpu.float().numpy()
    wf = lin_weight_for_oracle(lin, g)
    pw, sw, gw = o.quantize_weight(wf)
    assert np.array_equal(packed.cpu().numpy(), pw)
    assert np.array_equal(layout_to_canonical(inv_scale.cpu().numpy(), lin.n, lin.k), sw)
    r = o.nvfp4_linear_inference(xf, pw, sw, gw, None if bias is None else bias.float().numpy(), global_sf_x, g)
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(out_gpu.float().cpu().numpy(), r["out"], bound)
    return r


def lin_weight_for_oracle(lin, g):
    w = lin.w.float().numpy()
    return o.fold_weight(w, g) if g else w


@pytest.mark.parametrize("mode", ["dynamic", "static", "unit"])
def test_tiny_linear_end_to_end(mode):
    lin = workloads.tiny_linear()
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), lin.bias.to(DEV), act_scale=mode, input_amax=25.0)
    out = layer(lin.x.to(DEV))
    gsf_x = {"dynamic": None, "unit": np.float32(1.0),
             "static": np.float32(np.float32(2688.0) / np.float32(25.0))}[mode]
    r = check_against_oracle(lin, lin.x, out, layer.packed, layer.inv_scale, layer.global_sf_w, gsf_x, 0, lin.bias)
    codes, scales, used = nv().quantize_activation(lin.x.to(DEV), layer.activation_global_sf())
    assert np.array_equal(codes.cpu().numpy(), r["codes"])
    assert np.float32(used.item()) == r["gsf_x"]


def test_leading_dims_are_flattened():
    lin = workloads.tiny_linear()
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), lin.bias.to(DEV))
    x = lin.x.to(DEV)
    out3 = layer(x.reshape(4, 16, lin.k))
    assert out3.shape == (4, 16, lin.n)
    assert torch.equal(out3.reshape(-1, lin.n), layer(x))


def test_empty_input():
    lin = workloads.tiny_linear()
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None)
    out = layer(torch.empty((0, lin.k), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (0, lin.n)


def test_repeated_calls_are_bitwise_identical():
    lin = workloads.qwen3_attention(m=512)[1]
    w = lin.w.to(DEV)
    packed, inv_scale, gsf_w = nv().quantize_weight(w)
    x = lin.x.to(DEV)
    a = nv().nvfp4_linear(x, packed, inv_scale, gsf_w, None, lin.n)
    b = nv().nvfp4_linear(x, packed, inv_scale, gsf_w, None, lin.n)
    assert torch.equal(a, b)


@pytest.mark.parametrize("which", ["qkv", "fc_in", "fc_out"])
def test_vit_tiles_with_rotation(which):
    """Decoder linears with the group-16 block rotation folded into the weight and
    applied to each tile at run time; one dynamic scale per tile."""
    lin = workloads.vit_decoder_tiles(tiles=2, which=(which,))[0]
    g = lin.rotation_group
    rows = lin.meta["tile_rows"]
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=g)
    wf = o.fold_weight(lin.w.float().numpy(), g)
    pw, sw, gw = o.quantize_weight(wf)
    assert np.array_equal(layer.packed.cpu().numpy(), pw)
    x = lin.x.to(DEV)
    for t in range(lin.meta["tiles"]):
        tile = x[t * rows:(t + 1) * rows]
        out = layer(tile)
        # fusion contract: rotate inside == rotate first, then an unrotated linear
        xr = nv().rotate_activation(tile, g)
        split = nv().nvfp4_linear(xr, layer.packed, layer.inv_scale, layer.global_sf_w, None, lin.n)
        assert torch.equal(out, split)
        # oracle on a row sample of the tile
        sample = np.arange(0, rows, 61)
        xf = o.rotate_activation(lin.x[t * rows:(t + 1) * rows].float().numpy(), g)
        gx = o.global_sf(o.amax(xf))
        nib, s8 = o.nvfp4_quantize(xf[sample], gx)
        alpha = o.alpha_of(gx, gw)
        ref = o.nvfp4_gemm(o.pack_codes(nib), s8, pw, sw, alpha)
        bound = accumulation_bound(o.dequantize(o.pack_codes(nib), s8), o.dequantize(pw, sw), alpha)
        assert_gemm_close(out[torch.from_numpy(sample).to(DEV)].float().cpu().numpy(), ref, bound)


def test_per_tile_contract():
    """A tile decoded inside the tile loop equals the same tile decoded alone, bit for bit;
    one call over all tiles uses one amax for the batch, so with a dynamic scale it is
    not the per-tile result (why dynamic-scale decoders decode per tile)."""
    lin = workloads.vit_decoder_tiles(tiles=8, tokens=1024, which=("fc_in",))[0]
    rows = lin.meta["tile_rows"]
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=lin.rotation_group)
    x = lin.x.to(DEV)
    per_tile = [layer(x[t * rows:(t + 1) * rows]) for t in range(8)]
    alone = layer(x[3 * rows:4 * rows].clone())
    assert torch.equal(per_tile[3], alone)
    batched = layer(x)
    assert not torch.equal(torch.cat(per_tile), batched)
    # with a static scale, batching is the same as per tile
    st = nv().NVFP4Linear(layer.packed, layer.inv_scale, layer.global_sf_w, None, lin.k, lin.rotation_group,
                          "static", 40.0)
    assert torch.equal(torch.cat([st(x[t * rows:(t + 1) * rows]) for t in range(8)]), st(x))


def test_binding_rejects_bad_arguments():
    lin = workloads.tiny_linear()
    packed, inv_scale, gsf_w = nv().quantize_weight(lin.w.to(DEV))
    x = lin.x.to(DEV)
    with pytest.raises(ValueError, match="packed NVFP4 weight"):
        nv().nvfp4_linear(x, packed[:, :64].contiguous(), inv_scale, gsf_w, None, lin.n)
    with pytest.raises(ValueError, match="divisible by 16"):
        nv().nvfp4_linear(x[:, :200].contiguous(), packed[:, :100].contiguous(), inv_scale, gsf_w, None, lin.n)
    with pytest.raises(ValueError, match="rotation group"):
        nv().nvfp4_linear(x, packed, inv_scale, gsf_w, None, lin.n, rotation_group=12)
    with pytest.raises(ValueError, match="activation-scale mode"):
        nv().NVFP4Linear(packed, inv_scale, gsf_w, None, lin.k, None, "bogus")
    with pytest.raises(ValueError):
        nv().NVFP4Linear.from_weight(torch.zeros((8, 24), device=DEV, dtype=torch.bfloat16))


_DECODE_WEIGHTS = {}


def _decode_weight(name):
    """GPU-quantized decode-sweep weight (quantized once per projection)."""
    if name not in _DECODE_WEIGHTS:
        w = workloads.small_m_weight(name)
        packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
        _DECODE_WEIGHTS.clear()            # keep one projection's weight resident at a time
        _DECODE_WEIGHTS[name] = (w, packed, inv_scale, gsf_w)
    return _DECODE_WEIGHTS[name]


@pytest.mark.parametrize("m", [1, 16, 128])
@pytest.mark.parametrize("name", [p[0] for p in workloads.QWEN3_PROJECTIONS])
def test_decode_sweep_sampled_columns(name, m):
    """The small-M sweep through nvfp4_linear in the launch configuration the decode
    benchmark uses: every output row, on 160 sampled output columns (plus the last 16),
    against the oracle; the sampled weight rows' codes and scales must be bit-exact."""
    print(f"[decode sweep] M={m} {name}", flush=True)
    w, packed, inv_scale, gsf_w = _decode_weight(name)
    n, k = w.shape
    x = workloads.small_m_input(m, name)
    out = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, None, n)
    torch.cuda.synchronize()
    rng = np.random.default_rng(m * 100 + n)
    cols = np.unique(np.concatenate([rng.choice(n, 160, replace=False), np.arange(n - 16, n)]))
    wf = w.float().numpy()
    gw = o.global_sf(o.amax(wf))
    assert np.float32(gsf_w.item()) == gw
    nib, sw = o.nvfp4_quantize(wf[cols], gw)
    pw = o.pack_codes(nib)
    assert np.array_equal(packed[torch.from_numpy(cols).to(DEV)].cpu().numpy(), pw)
    r = o.nvfp4_linear_inference(x.float().numpy(), pw, sw, gw, None)
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(out.float().cpu().numpy()[:, cols], r["out"], bound)


@pytest.mark.parametrize("name", [p[0] for p in workloads.QWEN3_PROJECTIONS])
def test_decode_sweep_static_one_row(name):
    """One row of the small-M sweep with a static scale below the row's abs-max (some
    blocks saturate): the single-launch linear at full size, on 160 sampled output
    columns (plus the last 16) against the oracle."""
    print(f"[decode sweep, static] M=1 {name}", flush=True)
    w, packed, inv_scale, gsf_w = _decode_weight(name)
    n, k = w.shape
    x = workloads.small_m_input(1, name)
    xf = x.float().numpy()
    gx = o.global_sf(np.float32(0.8) * o.amax(xf))
    gxt = torch.tensor(float(gx), dtype=torch.float32, device=DEV)
    out = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, None, n, gxt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7 * n + k)
    cols = np.unique(np.concatenate([rng.choice(n, 160, replace=False), np.arange(n - 16, n)]))
    wf = w.float().numpy()
    gw = o.global_sf(o.amax(wf))
    nib, sw = o.nvfp4_quantize(wf[cols], gw)
    pw = o.pack_codes(nib)
    r = o.nvfp4_linear_inference(xf, pw, sw, gw, None, gx)
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(out.float().cpu().numpy()[:, cols], r["out"], bound)


def _segmented_inputs(segments, seg_rows, k, seed):
    """Row blocks with very different magnitudes, so per-segment scales differ."""
    x = workloads.draw("t3", (segments * seg_rows, k), seed, 0)
    scale = torch.tensor([2.0 ** (3 * s - 4) * (1.0 + 0.1 * s) for s in range(segments)]).repeat_interleave(seg_rows)
    return (x.float() * scale[:, None]).to(torch.bfloat16)


@pytest.mark.parametrize("segments,seg_rows,k,g", [(5, 37, 272, 16), (8, 64, 1024, 0), (3, 1, 96, 2), (16, 130, 512, 128)])
def test_segmented_quantize_equals_per_segment_calls(segments, seg_rows, k, g):
    """One global scale per row block: codes, scales and scales bit-identical to quantizing
    each block alone, and to the oracle."""
    x = _segmented_inputs(segments, seg_rows, k, segments * 7 + k)
    codes, scales, gsf = nv().quantize_activation_segmented(x.to(DEV), segments, g)
    codes_c = codes.cpu().numpy()
    scales_c = layout_to_canonical(scales.cpu().numpy(), segments * seg_rows, k)
    for s in range(segments):
        rows = slice(s * seg_rows, (s + 1) * seg_rows)
        c1, s1, g1 = nv().quantize_activation(x[rows].to(DEV).contiguous(), None, g)
        assert np.array_equal(codes_c[rows], c1.cpu().numpy())
        assert np.array_equal(scales_c[rows], layout_to_canonical(s1.cpu().numpy(), seg_rows, k))
        assert gsf[s].item() == g1.item()
        xf = x[rows].float().numpy()
        if g:
            xf = o.rotate_activation(xf, g)
        gx = o.global_sf(o.amax(xf))
        nib, s8 = o.nvfp4_quantize(xf, gx)
        assert np.float32(gsf[s].item()) == gx
        assert np.array_equal(codes_c[rows], o.pack_codes(nib))
        assert np.array_equal(scales_c[rows], s8)


@pytest.mark.parametrize("segments,seg_rows,k,n", [
    (4, 8, 1024, 1000),      # weight streaming (32 rows)
    (3, 40, 272, 300),       # K % 32 == 16: register-staged kernel
    (4, 256, 1024, 1536),    # pipelined kernel, segments aligned to tiles
    (3, 300, 2048, 4352),    # pipelined kernel, segments crossing tiles, split-K tail
])
def test_segmented_linear_per_tile_scales(segments, seg_rows, k, n):
    """nvfp4_linear_segmented on every GEMM kernel: each row block matches the oracle run
    on that block alone (its own dynamic scale), and the reported scales are the blocks'."""
    x = _segmented_inputs(segments, seg_rows, k, n + k)
    w = workloads.draw("normal", (n, k), 11, n, 0.02)
    bias = workloads.draw("normal", (n,), 12, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    gsf_out = torch.empty((segments,), dtype=torch.float32, device=DEV)
    out = nv().nvfp4_linear_segmented(x.to(DEV), segments, packed, inv_scale, gsf_w, bias.to(DEV), n, gsf_out=gsf_out)
    torch.cuda.synchronize()
    wf = w.float().numpy()
    pw, sw, gw = o.quantize_weight(wf)
    got = out.float().cpu().numpy()
    for s in range(segments):
        rows = slice(s * seg_rows, (s + 1) * seg_rows)
        r = o.nvfp4_linear_inference(x[rows].float().numpy(), pw, sw, gw, bias.float().numpy())
        assert np.float32(gsf_out[s].item()) == r["gsf_x"]
        bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
        assert_gemm_close(got[rows], r["out"], bound)


def test_segmented_vit_tiles_match_per_tile_calls():
    """The ViT decoder tiles (rotation g=16 folded into W, Student-t activations): one
    segmented pass over 8 tiles against the layer called on each tile alone."""
    lin = workloads.vit_decoder_tiles(tiles=8, tokens=1024, which=("fc_out",))[0]
    rows = lin.meta["tile_rows"]
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=lin.rotation_group)
    x = lin.x.to(DEV)
    batched = layer.forward_tiles(x, 8)
    for t in range(8):
        alone = layer(x[t * rows:(t + 1) * rows])
        bound = np.full(alone.shape, 0.0, dtype=np.float32)
        assert_gemm_close(batched[t * rows:(t + 1) * rows].float().cpu().numpy(), alone.float().cpu().numpy(), bound)


@pytest.mark.parametrize("rows,k,g", [(1, 16, 0), (37, 272, 16), (300, 1024, 0), (64, 512, 128)])
def test_amax_and_accumulate(rows, k, g):
    """Calibration abs-max of the (rotated) input: exact against the oracle; the
    accumulating form keeps the running maximum over batches."""
    xs = [workloads.draw("t3", (rows, k), rows + k, i, 1.0 + i) for i in range(3)]
    ref = []
    for x in xs:
        xf = x.float().numpy()
        ref.append(o.amax(o.rotate_activation(xf, g) if g else xf))
    first = nv().amax(xs[0].to(DEV), g)
    assert np.float32(first.item()) == np.float32(ref[0])
    running = torch.zeros((), dtype=torch.float32, device=DEV)
    for x in xs:
        nv().amax(x.to(DEV), g, out=running, accumulate=True)
    assert np.float32(running.item()) == np.float32(max(ref))


@pytest.mark.parametrize("amax", [0.0, 1e-13, 3.0e-5, 25.0, 448.0, 1.0e30])
@pytest.mark.parametrize("margin", [1.0, 1.25, 0.5])
def test_static_global_scale(amax, margin):
    a = torch.tensor(amax, dtype=torch.float32, device=DEV)
    got = np.float32(nv().static_global_sf(a, margin).item())
    assert got == o.global_sf(np.float32(np.float32(amax) * np.float32(margin)))


def test_calibration_then_static_forward():
    """calibrate_static_scales over three batches (rotation 16, margin 1.5): the static
    scale is 2688 / (largest recorded abs-max * 1.5), and the static forward matches the
    oracle run with that scale."""
    lin = workloads.vit_decoder_tiles(tiles=3, tokens=256, which=("qkv",))[0]
    rows = lin.meta["tile_rows"]
    g = lin.rotation_group
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=g)
    x = lin.x.to(DEV)
    n = nv().calibrate_static_scales([layer], lambda: [layer(x[t * rows:(t + 1) * rows]) for t in range(3)], 1.5)
    assert n == 1 and layer.act_scale == "static"
    xf = lin.x.float().numpy()
    recorded = max(o.amax(o.rotate_activation(xf[t * rows:(t + 1) * rows], g)) for t in range(3))
    gx = o.global_sf(np.float32(np.float32(recorded) * np.float32(1.5)))
    assert np.float32(layer.activation_global_sf().item()) == gx
    tile = x[:rows]
    out = layer(tile)
    check_against_oracle(lin, lin.x[:rows], out, layer.packed, layer.inv_scale, layer.global_sf_w, gx, g)


@pytest.mark.parametrize("m", [1, 5, 16])
@pytest.mark.parametrize("n,k", [(1024, 5120), (300, 4128), (5120, 1024)])
def test_static_decode_fused_quantize(m, n, k):
    """Static scale, up to 16 rows (one row in a single launch, more rows through the
    quantize pass's fp16 operand form): bit-identical to quantizing first and running
    nvfp4_gemm, and within tolerance of the oracle.  The scale saturates some blocks
    (static range below the true amax)."""
    x = workloads.draw("t3", (m, k), m + k, 0, 2.0)
    w = workloads.draw("normal", (n, k), 31, n, 0.02)
    bias = workloads.draw("normal", (n,), 32, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    xf = x.float().numpy()
    gx = o.global_sf(np.float32(0.5) * o.amax(xf))
    gxt = torch.tensor(float(gx), dtype=torch.float32, device=DEV)
    fused = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, bias.to(DEV), n, gxt)
    codes, scales, _ = nv().quantize_activation(x.to(DEV), gxt)
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, gxt, gsf_w, bias.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    pw, sw, gw = o.quantize_weight(w.float().numpy())
    r = o.nvfp4_linear_inference(xf, pw, sw, gw, bias.float().numpy(), gx)
    assert np.array_equal(codes.cpu().numpy(), r["codes"])
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(fused.float().cpu().numpy(), r["out"], bound)


@pytest.mark.parametrize("n,k", [(5120, 25600), (25600, 5120), (1024, 5120), (64, 16384), (8, 32), (17, 96),
                                 (300, 1568), (4096, 49152), (5120, 16384), (5120, 16640)])
def test_static_one_row_fused_decode(n, k):
    """Static scale, one row: the decode GEMM's waves quantize their own K ranges of the row
    (one launch).  Bit-identical to quantizing first and running nvfp4_gemm, codes equal to
    the oracle's; K spans one super tile up to ranges too long for one wave's region (those
    shapes take the two-launch path and must agree all the same)."""
    print(f"[static one-row fused decode] n={n} k={k}", flush=True)
    x = workloads.draw("t3", (1, k), k, 1, 2.0)
    w = workloads.draw("normal", (n, k), 33, n, 0.02)
    bias = workloads.draw("normal", (n,), 34, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    xf = x.float().numpy()
    gx = o.global_sf(np.float32(0.75) * o.amax(xf))
    gxt = torch.tensor(float(gx), dtype=torch.float32, device=DEV)
    fused = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, bias.to(DEV), n, gxt)
    codes, scales, _ = nv().quantize_activation(x.to(DEV), gxt)
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, gxt, gsf_w, bias.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    nib, s8 = o.nvfp4_quantize(xf, gx)
    assert np.array_equal(codes.cpu().numpy(), o.pack_codes(nib))
    assert np.array_equal(layout_to_canonical(scales.cpu().numpy(), 1, k), s8)


@pytest.mark.parametrize("n,k", [(5120, 25600), (25600, 5120), (1024, 5120), (64, 16384), (8, 32), (17, 96),
                                 (300, 1568), (4096, 49152), (5120, 16384), (5120, 16640)])
def test_dynamic_one_row_fused_decode(n, k):
    """Dynamic scale, one row: every decode block takes the row's abs-max itself, then its
    waves quantize their K ranges (one launch).  Bit-identical to the dynamic quantize then
    nvfp4_gemm; the scale used (reported through the segmented call) and the codes equal
    the oracle's."""
    print(f"[dynamic one-row fused decode] n={n} k={k}", flush=True)
    x = workloads.draw("t3", (1, k), k, 2, 2.0)
    w = workloads.draw("normal", (n, k), 35, n, 0.02)
    bias = workloads.draw("normal", (n,), 36, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    xd = x.to(DEV)
    fused = nv().nvfp4_linear(xd, packed, inv_scale, gsf_w, bias.to(DEV), n)
    codes, scales, gsf = nv().quantize_activation(xd, None)
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, gsf, gsf_w, bias.to(DEV))
    used = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    seg = nv().nvfp4_linear_segmented(xd, 1, packed, inv_scale, gsf_w, bias.to(DEV), n, gsf_out=used)
    torch.cuda.synchronize()
    assert torch.equal(fused, two) and torch.equal(seg, fused)
    xf = x.float().numpy()
    gx = o.global_sf(o.amax(xf))
    assert np.float32(gsf.item()) == gx and np.float32(used.item()) == gx
    nib, s8 = o.nvfp4_quantize(xf, gx)
    assert np.array_equal(codes.cpu().numpy(), o.pack_codes(nib))
    assert np.array_equal(layout_to_canonical(scales.cpu().numpy(), 1, k), s8)


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("n,k", [(1024, 5120), (64, 16384), (5120, 8192)])
def test_one_row_fused_decode_without_bias(n, k, static):
    """The one-launch linear without a bias (split and unsplit plans, four- and eight-wave
    blocks) equals the quantize pass plus nvfp4_gemm bit for bit, and the oracle within
    the GEMM tolerance."""
    x = workloads.draw("normal", (1, k), k, 3, 1.0)
    w = workloads.draw("normal", (n, k), 39, n, 0.02)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    xf = x.float().numpy()
    gx = o.global_sf(np.float32(0.9) * o.amax(xf)) if static else None
    gxt = None if gx is None else torch.tensor(float(gx), dtype=torch.float32, device=DEV)
    fused = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, None, n, gxt)
    codes, scales, used = nv().quantize_activation(x.to(DEV), gxt)
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, used, gsf_w, None)
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    pw, sw, gw = o.quantize_weight(w.float().numpy())
    r = o.nvfp4_linear_inference(xf, pw, sw, gw, None, gx)
    assert np.array_equal(codes.cpu().numpy(), r["codes"])
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(fused.float().cpu().numpy(), r["out"], bound)


@pytest.mark.parametrize("n,k", [(1024, 5120), (64, 16384)])
def test_dynamic_one_row_fused_decode_zero_row(n, k):
    """An all-zero row takes the floored scale and gives the bias alone, as the oracle."""
    x = torch.zeros((1, k), dtype=torch.bfloat16)
    w = workloads.draw("normal", (n, k), 37, n, 0.02)
    bias = workloads.draw("normal", (n,), 38, n, 0.01)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    used = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    out = nv().nvfp4_linear_segmented(x.to(DEV), 1, packed, inv_scale, gsf_w, bias.to(DEV), n, gsf_out=used)
    torch.cuda.synchronize()
    assert np.float32(used.item()) == o.global_sf(np.float32(0.0))
    pw, sw, gw = o.quantize_weight(w.float().numpy())
    r = o.nvfp4_linear_inference(x.float().numpy(), pw, sw, gw, bias.float().numpy())
    assert np.array_equal(out.float().cpu().numpy(), r["out"])


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("static,g", [(False, 0), (True, 0), (False, 16), (True, 16)])
@pytest.mark.parametrize("n,k", [(1000, 4128), (5120, 1024)])
def test_fp16_activation_decode_equals_codes_path(m, static, g, n, k):
    """At most four rows nvfp4_linear hands the decode GEMM the quantized activation in
    its fp16 operand form (code * scale * 2^-8) instead of codes and scales: the same
    operands, so the output is bit-identical to quantizing first and running nvfp4_gemm,
    and within tolerance of the oracle (partial last K tile with K = 4128)."""
    x = workloads.draw("t3", (m, k), 7 * m + k, 0, 2.0)
    w = workloads.draw("normal", (n, k), 41, n, 0.02)
    bias = workloads.draw("normal", (n,), 42, n, 0.01)
    # with a rotation the weight carries it, folded offline (bf16-exact values)
    wf = o.fold_weight(w.float().numpy(), g) if g else w.float().numpy()
    w_dev = torch.from_numpy(np.ascontiguousarray(wf, dtype=np.float32)).to(torch.bfloat16).to(DEV)
    packed, inv_scale, gsf_w = nv().quantize_weight(w_dev)
    xf = x.float().numpy()
    gx = o.global_sf(o.amax(xf)) if static else None
    gxt = None if gx is None else torch.tensor(float(gx), dtype=torch.float32, device=DEV)
    out = nv().nvfp4_linear(x.to(DEV), packed, inv_scale, gsf_w, bias.to(DEV), n, gxt, g)
    codes, scales, used = nv().quantize_activation(x.to(DEV), gxt, g)
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, used, gsf_w, bias.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    pw, sw, gw = o.quantize_weight(wf)
    r = o.nvfp4_linear_inference(xf, pw, sw, gw, bias.float().numpy(), gx, g)
    assert np.array_equal(codes.cpu().numpy(), r["codes"])
    bound = accumulation_bound(o.dequantize(r["codes"], r["scales"]), o.dequantize(pw, sw), r["alpha"])
    assert_gemm_close(out.float().cpu().numpy(), r["out"], bound)


@pytest.mark.parametrize("m", [1, 3])
def test_fp16_activation_decode_swiglu(m):
    """The SwiGLU linear at few rows takes the same fp16-activation decode path:
    bit-identical to quantizing the product and running nvfp4_gemm."""
    n, k = 640, 1024
    gate = workloads.draw("normal", (m, k), 51 + m, 0, 1.0)
    up = workloads.draw("normal", (m, k), 61 + m, 0, 1.0)
    w = workloads.draw("normal", (n, k), 71, n, 0.02)
    packed, inv_scale, gsf_w = nv().quantize_weight(w.to(DEV))
    out = nv().nvfp4_linear_swiglu(gate.to(DEV), up.to(DEV), packed, inv_scale, gsf_w, None, n)
    codes, scales, used = nv().quantize_swiglu(gate.to(DEV), up.to(DEV))
    two = nv().nvfp4_gemm(codes, scales, packed, inv_scale, used, gsf_w, None)
    torch.cuda.synchronize()
    assert torch.equal(out, two)


@pytest.mark.slow
@pytest.mark.parametrize("which", ["qkv", "fc_in", "fc_out"])
def test_segmented_vit_tiles_full_size(which):
    """The ViT decoder batch at its configured size, in the call bench.py times: 8 tiles x
    4096 tokens through nvfp4_linear_segmented with the group-16 rotation.  Every tile's
    global scale is bit-exact against the oracle's (rotated amax of that tile alone); on
    sampled rows of every tile the codes and scales of the segmented quantizer are
    bit-exact and the outputs are within the GEMM tolerance of the oracle."""
    lin = workloads.vit_decoder_tiles(tiles=8, which=(which,))[0]
    g, rows, tiles = lin.rotation_group, lin.meta["tile_rows"], lin.meta["tiles"]
    print(f"segmented full size: {which} {tiles} x [{rows}, {lin.k}] x [{lin.n}, {lin.k}] rot{g}", flush=True)
    wd = nv().rotate_activation(lin.w.to(DEV).float(), g, out_dtype=torch.bfloat16)
    packed, inv_scale, gsf_w = nv().quantize_weight(wd)
    x = lin.x.to(DEV)
    gsf_out = torch.empty((tiles,), dtype=torch.float32, device=DEV)
    out = nv().nvfp4_linear_segmented(x, tiles, packed, inv_scale, gsf_w, None, lin.n, g, gsf_out=gsf_out)
    codes, scales, gsf_q = nv().quantize_activation_segmented(x, tiles, g)
    torch.cuda.synchronize()
    assert torch.equal(gsf_out, gsf_q)
    pw, sw, gw = o.quantize_weight(o.fold_weight(lin.w.float().numpy(), g))
    assert np.array_equal(packed.cpu().numpy(), pw) and np.float32(gsf_w.item()) == gw
    codes_c = codes.cpu().numpy()
    scales_c = layout_to_canonical(scales.cpu().numpy(), tiles * rows, lin.k)
    got = out.float().cpu().numpy()
    xall = lin.x.float().numpy()
    for t in range(tiles):
        xt = o.rotate_activation(xall[t * rows:(t + 1) * rows], g)
        gx = o.global_sf(o.amax(xt))
        assert np.float32(gsf_out[t].item()) == gx, t
        sample = np.arange(t % 7, rows, 257)
        nib, s8 = o.nvfp4_quantize(xt[sample], gx)
        assert np.array_equal(codes_c[t * rows + sample], o.pack_codes(nib)), t
        assert np.array_equal(scales_c[t * rows + sample], s8), t
        alpha = o.alpha_of(gx, gw)
        ref = o.nvfp4_gemm(o.pack_codes(nib), s8, pw, sw, alpha)
        bound = accumulation_bound(o.dequantize(o.pack_codes(nib), s8), o.dequantize(pw, sw), alpha)
        assert_gemm_close(got[t * rows + sample], ref, bound)


def test_calibration_block_and_errors():
    """calibration(): inside the block the layer runs dynamic numerics and records; a block
    that raises leaves the layer dynamic; a layer that saw no input is an error."""
    lin = workloads.vit_decoder_tiles(tiles=2, tokens=128, which=("qkv",))[0]
    g = lin.rotation_group
    layer = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=g)
    x = lin.x.to(DEV)
    with nv().calibration([layer], margin=1.25):
        assert layer.calibrating
        inside = layer(x[:128])
    assert not layer.calibrating and layer.act_scale == "static"
    assert torch.equal(inside, nv().nvfp4_linear(x[:128], layer.packed, layer.inv_scale, layer.global_sf_w, None,
                                                 lin.n, None, g))
    rec = o.amax(o.rotate_activation(lin.x[:128].float().numpy(), g))
    assert np.float32(layer.activation_global_sf().item()) == o.global_sf(np.float32(rec) * np.float32(1.25))
    fresh = nv().NVFP4Linear.from_weight(lin.w.to(DEV), None, rotation_group=g)
    with pytest.raises(KeyError):
        with nv().calibration([fresh]):
            fresh(x[:128])
            raise KeyError("stop")
    assert not fresh.calibrating and fresh.act_scale == "dynamic"
    with pytest.raises(RuntimeError, match="no nonzero activation"):
        with nv().calibration([fresh]):
            pass
    assert fresh.act_scale == "dynamic"
