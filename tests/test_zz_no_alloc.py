"""fa_fwd_noalloc against fa_fwd_ws through the C ABI.

fa_fwd_noalloc runs the same kernels as fa_fwd_ws, with the key-split partials
in the library's static per-GPU scratch instead of a caller workspace, so its
outputs must equal fa_fwd_ws's bit for bit. Two split calls in a row, the second
on a smaller input (the scratch then holds the first call's partials beyond the
second's), then a call that needs no scratch. The first call is also checked
against the FP64 oracle on sampled rows.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from gpu_helpers import check_lse, check_o, have_gpu, to_dev, to_f64
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _run(lib, entry, q, k, v, causal, scale, ws=None):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
            int(causal), float(scale)]
    if entry == "fa_fwd_ws":
        st = lib.fa_fwd_ws(*args, ws.data_ptr() if ws is not None else None,
                           ws.numel() if ws is not None else 0, stream)
    else:
        st = lib.fa_fwd_noalloc(*args, stream)
    assert st == 0, f"{entry}: {lib.fa_status_string(st).decode()}"
    return o, lse


CASES = [
    si.FwdCase("noalloc 1x1x8192 d128", 1, 1, 1, 8192, 128, False, seed=2, sampled_rows=256),
    si.FwdCase("noalloc 1x2x2000 d64 causal gqa", 1, 2, 1, 2000, 64, True, seed=21),
    si.FwdCase("noalloc 1x4x960 d128 gqa (no split)", 1, 4, 2, 960, 128, False, seed=22),
]


def test_noalloc_matches_fwd_ws_on_consecutive_calls():
    from exact_tiled_attention_fa_amd import _lib
    lib = _lib.lib()
    assert lib.fa_fwd_noalloc_max_scratch_bytes() == 34 << 20
    for n, case in enumerate(CASES):
        print(f"[noalloc] {case.name} causal={case.causal} seed={case.seed}", flush=True)
        sys.stdout.flush()
        qb, kb, vb = si.fwd_inputs(case)
        q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
        wsb = lib.fa_fwd_workspace_bytes(case.B, case.Hq, case.N, case.d)
        assert (wsb > 0) == (n < 2), "the first two shapes split their keys, the last one does not"
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0") if wsb else None
        o_ref, lse_ref = _run(lib, "fa_fwd_ws", q, k, v, case.causal, case.scale, ws)
        o_na, lse_na = _run(lib, "fa_fwd_noalloc", q, k, v, case.causal, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), f"{case.name}: O differs"
        assert torch.equal(lse_na.view(torch.int32), lse_ref.view(torch.int32)), f"{case.name}: lse differs"
        if n == 0:
            rows = np.stack([si.sample_rows(case.seed, h, case.N, case.sampled_rows) for h in range(case.Hq)])
            qf, kf, vf = (si.bf16_bits_to_f32(x) for x in (qb, kb, vb))
            vx = np.concatenate([vf, np.abs(vf)], axis=-1)
            ox, lr = fa_oracle.attention_ref(qf, kf, vx, case.causal, case.scale, rows=rows)
            o_np = np.stack([to_f64(o_na)[:, h, rows[h]] for h in range(case.Hq)], axis=1)
            l_np = np.stack([to_f64(lse_na)[:, h, rows[h]] for h in range(case.Hq)], axis=1)
            check_o(o_np, ox[..., :case.d], ox[..., case.d:], case.name, split=True)
            check_lse(l_np, lr, case.name)
        del q, k, v, ws, o_ref, lse_ref, o_na, lse_na
