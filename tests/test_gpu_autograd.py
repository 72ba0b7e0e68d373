"""torch.autograd wiring of the library's forward and backward passes.

The kernels' numerics are checked against the oracle in test_gpu_fwd.py and
test_gpu_bwd.py; here the differentiable entry point must return exactly what
the two C-ABI calls return (same kernels, same inputs), for a plain and a
non-contiguous upstream gradient.
"""
import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.mark.parametrize("causal", [False, True])
def test_attention_autograd_matches_abi_calls(causal):
    import torch
    import exact_tiled_attention_fa_amd as fa
    case = si.FwdCase("autograd", 1, 4, 2, 300, 128, causal, seed=51)
    print(f"[autograd] causal={causal} B1 Hq4 Hkv2 N300 d128 seed=51", flush=True)
    qb, kb, vb = si.fwd_inputs(case)
    q, k, v = (to_dev(x).requires_grad_(True) for x in (qb, kb, vb))
    g = to_dev(si.normal_bf16(np.random.default_rng(52), (1, 4, 300, 128)))
    o = fa.attention(q, k, v, causal=causal)
    o.backward(g)
    o_ref, lse_ref = fa.fwd(q.detach(), k.detach(), v.detach(), causal=causal)
    dq, dk, dv = fa.bwd(q.detach(), k.detach(), v.detach(), o_ref, lse_ref, g, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach().view(torch.int16), o_ref.view(torch.int16))
    for got, ref in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_attention_autograd_noncontiguous_gradient():
    import torch
    import exact_tiled_attention_fa_amd as fa
    case = si.FwdCase("autograd nc", 1, 2, 2, 130, 128, False, seed=53)
    print("[autograd] non-contiguous dO B1 Hq2 Hkv2 N130 d128 seed=53", flush=True)
    qb, kb, vb = si.fwd_inputs(case)
    q, k, v = (to_dev(x).requires_grad_(True) for x in (qb, kb, vb))
    gt = to_dev(si.normal_bf16(np.random.default_rng(54), (1, 2, 128, 130)))
    g = gt.transpose(2, 3)  # [1, 2, 130, 128], not contiguous
    o = fa.attention(q, k, v)
    o.backward(g)
    o_ref, lse_ref = fa.fwd(q.detach(), k.detach(), v.detach())
    dq, dk, dv = fa.bwd(q.detach(), k.detach(), v.detach(), o_ref, lse_ref, g.contiguous())
    torch.cuda.synchronize()
    for got, ref in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
