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
    with pytest.raises(ValueError, match="act_scale"):
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
