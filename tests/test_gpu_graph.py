"""The library's calls captured in a HIP graph and replayed.

The kernels allocate nothing and record no memory fills, so a captured
sequence (quantize, dequantize, GEMV, GEMM, a GEMV chain reusing its sync
buffer, the backward product) must give, on every replay, the bits of the
same calls run eagerly.  Outputs are overwritten with a different value
between replays, with eager work and synchronisations in between.
"""

import pytest
import torch

from bit_group_wise_amd import q4
from _helpers import DEV

pytestmark = pytest.mark.gpu


def _run(w, q, qdq, xs, x16, xm, dy, outs, chain, sync):
    q4.quantize(w, q4.NF4, 64, out=q)
    q4.quantize(w, q4.NF4_DQ, 32, out=qdq)
    q4.dequantize(q, torch.bfloat16, out=outs["deq"])
    q4.gemv(xs, q, out=outs["gemv"])
    q4.gemv(x16, qdq, out=outs["skinny"])
    q4.gemm(xm, q, out=outs["gemm"])
    q4.gemm_dx(dy, q, out=outs["dx"])
    q4.gemv_chain(chain, sync=sync)


def test_graph_replays_match_eager():
    N, K = 1536, 2048
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    w = torch.empty((N, K), dtype=torch.float16, device=DEV).normal_(0.0, 0.02, generator=gen)
    q = q4.alloc_quantized(q4.NF4, 64, N, K, DEV)
    qdq = q4.alloc_quantized(q4.NF4_DQ, 32, N, K, DEV)
    xs = torch.randn((1, K), generator=gen, device=DEV).to(torch.bfloat16)
    x16 = torch.randn((16, K), generator=gen, device=DEV).to(torch.bfloat16)
    xm = torch.randn((300, K), generator=gen, device=DEV).to(torch.bfloat16)
    dy = torch.randn((300, N), generator=gen, device=DEV).to(torch.bfloat16)
    outs = {
        "deq": torch.empty((N, K), dtype=torch.bfloat16, device=DEV),
        "gemv": torch.empty((1, N), dtype=torch.bfloat16, device=DEV),
        "skinny": torch.empty((16, N), dtype=torch.bfloat16, device=DEV),
        "gemm": torch.empty((300, N), dtype=torch.bfloat16, device=DEV),
        "dx": torch.empty((300, K), dtype=torch.bfloat16, device=DEV),
    }
    # a chain: two independent products and one reading the first's output
    ya = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
    yb = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
    q2 = q4.alloc_quantized(q4.NF4, 64, K, N, DEV)
    q4.quantize(torch.empty((K, N), dtype=torch.float16, device=DEV).normal_(0.0, 0.02,
                                                                            generator=gen),
                q4.NF4, 64, out=q2)
    yc = torch.empty((1, K), dtype=torch.bfloat16, device=DEV)
    chain = [(xs, q, ya, q4.TASK_NO_WAIT), (xs, q, yb, q4.TASK_NO_WAIT), (ya, q2, yc, 0)]
    outs_chain = [ya, yb, yc]
    sync = q4.chain_sync(DEV)

    def everything():
        return list(outs.values()) + outs_chain + [q.codes, q.scales, qdq.codes, qdq.scales]

    _run(w, q, qdq, xs, x16, xm, dy, outs, chain, sync)
    torch.cuda.synchronize()
    ref = [t.clone() for t in everything()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(w, q, qdq, xs, x16, xm, dy, outs, chain, sync)  # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(w, q, qdq, xs, x16, xm, dy, outs, chain, sync)

    for rep in range(3):
        for t in everything():
            t.view(torch.uint8).fill_(0x55 + rep)
        q4.dequantize(q2, torch.bfloat16)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(everything(), ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i}"
        assert not sync.any().item()
