"""fa_fwd_noalloc inside a captured HIP graph.

fa_fwd_noalloc is the entry point for callers that cannot allocate, graph
capture among them: it records only its kernel launches (the key-split
partials live in the library's static per-GPU scratch, and nothing is cleared
with a memset). The graph is captured on a key-split shape (forward kernel +
merge) and on a single-launch shape, then replayed several times with eager
work (other library calls that also use the scratch) and synchronisations in
between, after the inputs change in place; every replay must equal the eager
result bit for bit.
"""
import pytest
import torch

import seeded_inputs as si
from gpu_helpers import have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.mark.parametrize("shape,split", [((1, 1, 8192, 128, False), True), ((1, 2, 6000, 128, True), True),
                                         ((2, 32, 2048, 64, False), False)],
                         ids=["split", "split-causal", "single"])
def test_noalloc_forward_replays_in_a_graph(shape, split):
    import exact_tiled_attention_fa_amd as fa
    B, H, N, d, causal = shape
    print(f"[graph] fwd_noalloc B{B} H{H} N{N} d{d} causal={causal}", flush=True)
    assert (fa.fwd_workspace_bytes(B, H, N, d) > 0) == split
    cases = [si.FwdCase("graph", B, H, H, N, d, causal, seed=9500 + r + N) for r in range(3)]
    draws = [tuple(to_dev(x) for x in si.fwd_inputs(c)) for c in cases]
    q, k, v = (t.clone() for t in draws[0])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    # eager call first: resolves the scratch address and the CU count before capture
    fa.fwd_noalloc(q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fa.fwd_noalloc(q, k, v, o, lse, causal=causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = [tuple(to_dev(x) for x in si.fwd_inputs(si.FwdCase("graph other", 1, 1, 1, 8192, 128, True, seed=9600)))]
    for rep in range(5):
        src = draws[rep % len(draws)]
        for dst, s in zip((q, k, v), src):
            dst.copy_(s)
        # eager reference on fresh buffers (fa_fwd_ws: its own workspace)
        o_ref = torch.empty_like(q)
        l_ref = torch.empty_like(lse)
        fa.prepare_fwd(q, k, v, o_ref, l_ref, causal=causal)()
        # eager work between replays that also uses the static scratch
        oq, ok_, ov = other[0]
        o_x = torch.empty_like(oq)
        l_x = torch.empty((1, 1, 8192), dtype=torch.float32, device=oq.device)
        fa.fwd_noalloc(oq, ok_, ov, o_x, l_x, causal=True)
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"replay {rep}: O differs from eager"
        assert torch.equal(lse, l_ref), f"replay {rep}: lse differs from eager"
