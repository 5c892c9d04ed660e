"""HIP graph capture of the linear: every replay against an eager call on fresh inputs.

Each case captures one nvfp4_linear (or nvfp4_linear_noalloc) call on static input,
workspace and output buffers.  Then, three times: new values (and a new range, so the
dynamic scale changes) are copied into the static input, the graph is replayed, the same
call runs eagerly into a second output, and the two must agree bit for bit.  The cases
cover every kernel path of the linear: the one-row single launch (dynamic and static
scale, split and unsplit), the fp16-activation decode, the 16-row decode, the skinny GEMM,
the pipelined GEMM with its split-K tail, and the gate projection itself.  The library
issues no memset and no allocation inside a call, so the captured kernels are the eager
ones.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def nv():
    import nvfp4_w4a4_quantized_global_amd as m
    return m


CASES = [
    (1, 5120, 1024, None),       # one row, dynamic scale, single launch
    (1, 8192, 5120, 12.0),       # one row, static scale, eight-wave blocks
    (1, 25600, 5120, None),      # one row, dynamic scale on a long row: quantize pass + decode GEMM
    (3, 4096, 1024, None),       # fp16-activation decode
    (16, 5120, 1024, None),      # decode GEMM on codes
    (40, 5120, 3072, 8.0),       # skinny GEMM, static scale
    (1024, 5120, 3072, None),    # pipelined GEMM with a split-K tail
]


def _run_case(m, k, n, gsf_x, noalloc):
    lib = nv()
    print(f"[graph] m={m} k={k} n={n} gsf_x={gsf_x} noalloc={noalloc}", flush=True)
    w = workloads.draw("normal", (n, k), 51, n, 0.02).to(DEV)
    packed, inv_scale, gsf_w = lib.quantize_weight(w.to(torch.bfloat16))
    bias = workloads.draw("normal", (n,), 52, n, 0.01).to(DEV)
    gx = None if gsf_x is None else torch.tensor(gsf_x, dtype=torch.float32, device=DEV)
    x = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
    x.copy_(workloads.draw("t3", (m, k), 53, m, 1.0).to(DEV))
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    ws = None if noalloc else torch.empty((lib.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=DEV)

    def call(o):
        if noalloc:
            lib.nvfp4_linear_noalloc(x, packed, inv_scale, gsf_w, bias, n, gx, 0, out=o)
        else:
            lib.nvfp4_linear(x, packed, inv_scale, gsf_w, bias, n, gx, 0, ws, o)

    call(out)                        # one-time set-up (kernel attributes) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(out)
    torch.cuda.synchronize()
    ref = torch.empty_like(out)
    for r in range(3):
        x.copy_(workloads.draw("t3", (m, k), 54 + r, m, 1.0 + 2.0 * r).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {r} differs from the eager call"
        assert torch.isfinite(got.float()).all()


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("m,k,n,gsf_x", CASES)
def test_graph_replays_match_eager(m, k, n, gsf_x, noalloc):
    _run_case(m, k, n, gsf_x, noalloc)


@pytest.mark.slow
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager_gate_projection(noalloc):
    """The headline shape, x [4096, 5120] against W [25600, 5120], dynamic scale."""
    _run_case(4096, 5120, 25600, None, noalloc)
