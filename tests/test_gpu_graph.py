"""The linear chains (INT8 and FP8) captured in a HIP graph.

The library allocates, clears and synchronizes nothing inside its calls, so a
capture (torch.cuda.CUDAGraph on its capture stream) holds exactly the
chains' kernel launches: paired quantize passes, GEMMs that fold column
maxima in their prologue, contraction splits with their partial planes.
Each replay, with new inputs copied into the captured buffers by eager work
between replays, must equal the eager chains on the same inputs byte for
byte (the eager chains are checked against the oracle elsewhere), and the
eager calls made between replays must not disturb the graph's buffers.
"""
import pytest
import torch

from workloads import LinearShape, linear_inputs

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def same_bytes(a, b):
    return a.shape == b.shape and bool((a.view(torch.int16) == b.view(torch.int16)).all())


# (300, 264, 1000): ragged tiles; (1024, 1024, 8192): the forward's contraction
# split; (512, 4096, 1024): dY's row pass and W's column pass in one launch.
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("M,N,K", [(300, 264, 1000), (1024, 1024, 8192), (512, 4096, 1024)])
def test_linear_chains_replayed_from_a_hip_graph(rounding, M, N, K):
    shape = LinearShape("graph", M, N, K)
    dev = torch.device("cuda")
    t = linear_inputs(shape, seed=0, device=dev)
    X, W, dY = t["X"].clone(), t["W"].clone(), t["dY"].clone()
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(max(1, i8.linear_workspace_bytes(M, N, K, False)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, i8.linear_workspace_bytes(M, N, K, True)), dtype=torch.uint8, device=dev)
    seed, off = 17, 9 << 44

    def step():
        _, cx, cw = i8.linear_fwd_colmax(X, W, rounding, seed, off, out=Y, workspace=wsf)
        i8.linear_bwd(dY, X, W, rounding, seed, off, dX=dX, dW=dW, workspace=wsb, colmax_x=cx, colmax_w=cw)
        return cx, cw

    # one eager call first, on a side stream as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cx_g, cw_g = step()

    for rep in range(3):
        u = linear_inputs(shape, seed=rep + 1, device=dev)
        X.copy_(u["X"])
        W.copy_(u["W"])
        dY.copy_(u["dY"])
        g.replay()
        torch.cuda.synchronize()
        got = {"Y": Y.clone(), "dX": dX.clone(), "dW": dW.clone(), "cx": cx_g.clone(), "cw": cw_g.clone()}
        # the eager chains on the same inputs, into their own buffers
        Ye, cxe, cwe = i8.linear_fwd_colmax(X, W, rounding, seed, off)
        dXe, dWe = i8.linear_bwd(dY, X, W, rounding, seed, off, colmax_x=cxe, colmax_w=cwe)
        torch.cuda.synchronize()
        for name, a, b in (("Y", got["Y"], Ye), ("dX", got["dX"], dXe), ("dW", got["dW"], dWe)):
            assert same_bytes(a, b), f"replay {rep}: {name} differs from the eager chains"
        assert torch.equal(got["cx"].view(torch.int32), cxe.view(torch.int32)), f"replay {rep}: colmax X"
        assert torch.equal(got["cw"].view(torch.int32), cwe.view(torch.int32)), f"replay {rep}: colmax W"
    del g


@pytest.mark.parametrize("M,N,K", [(300, 264, 1000), (256, 512, 8192)])
def test_fp8_chains_replayed_from_a_hip_graph(M, N, K):
    """The FP8 chains (the second shape splits its forward contraction into
    fp32 planes) captured and replayed with new inputs: every replay equals
    the eager chains byte for byte."""
    shape = LinearShape("graph8", M, N, K)
    dev = torch.device("cuda")
    t = linear_inputs(shape, seed=0, device=dev)
    X, W, dY = t["X"].clone(), t["W"].clone(), t["dY"].clone()
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(max(1, i8.linear_workspace_bytes(M, N, K, False)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, i8.linear_workspace_bytes(M, N, K, True)), dtype=torch.uint8, device=dev)

    def step():
        _, cx, cw = i8.linear_fwd_fp8_colmax(X, W, out=Y, workspace=wsf)
        i8.linear_bwd_fp8(dY, X, W, workspace=wsb, dX=dX, dW=dW, colmax_x=cx, colmax_w=cw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        u = linear_inputs(shape, seed=rep + 1, device=dev)
        X.copy_(u["X"])
        W.copy_(u["W"])
        dY.copy_(u["dY"])
        g.replay()
        torch.cuda.synchronize()
        got = (Y.clone(), dX.clone(), dW.clone())
        Ye, cxe, cwe = i8.linear_fwd_fp8_colmax(X, W)
        dXe, dWe = i8.linear_bwd_fp8(dY, X, W, colmax_x=cxe, colmax_w=cwe)
        torch.cuda.synchronize()
        for name, a, b in zip(("Y", "dX", "dW"), got, (Ye, dXe, dWe)):
            assert same_bytes(a, b), f"replay {rep}: {name} differs from the eager chains"
    del g
