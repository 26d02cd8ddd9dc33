"""The GEMM under HIP graph capture: the library launches only on the caller's stream and
allocates nothing, so a torch CUDA graph can capture its calls.  Every replay is checked
against the eager result for the inputs the replay read, with eager work and
synchronisations between the replays."""
import pytest
import torch

import dense_fp16_gemm_fp32_amd as g
import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,epi", [((256, 256, 256), "none"), ((1000, 3000, 777), "bias_gelu"),
                                       ((2048, 2047, 2048), "bias_gelu"), ((64, 5, 200), "bias")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_captured_gemm_replays_match_eager_calls(shape, epi):
    """2048 x 2047 takes a direct launch plus a narrow one, 64 x 5 the narrow kernel alone:
    both launches of a call land in the graph."""
    M, N, K = shape
    print("graph", shape, epi, flush=True)
    dev = torch.device("cuda:0")
    A, B, bias = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=11)
    sA, sB, sbias = A.to(dev), B.to(dev), bias.to(dev)
    b_arg = sbias if epi != "none" else None
    out = torch.empty((M, N), dtype=torch.float16, device=dev)
    # warm the stream up outside the capture, as torch's graph API asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.gemm(sA, sB, b_arg, epi, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.gemm(sA, sB, b_arg, epi, out=out)

    for replay in range(3):
        A2, B2, bias2 = workloads.make_inputs(M, N, K, "uniform", with_bias=True, seed=100 + replay)
        sA.copy_(A2.to(dev))
        sB.copy_(B2.to(dev))
        sbias.copy_(bias2.to(dev))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        eager = g.gemm(sA, sB, b_arg, epi)          # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % replay
