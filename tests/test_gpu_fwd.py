"""GPU parity of the forward kernel against the FP64 oracle, through the C ABI.

Every workload's inputs come from seeded_inputs (the same BF16 values reach the
GPU and, widened exactly, the oracle). Large workloads are checked on a seeded
sample of rows per head; the kernel always computes every row.
"""
import math
import sys

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import check_lse, check_o, have_gpu, to_dev, to_f64
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _may_split(case) -> bool:
    """Whether the library may split this shape's keys (BF16 partials; either mask)."""
    import exact_tiled_attention_fa_amd as fa
    return fa.fwd_workspace_bytes(case.B, case.Hq, case.N, case.d) > 0


def _run_case(case: si.FwdCase, scale=None, extra_rows=()):
    import exact_tiled_attention_fa_amd as fa
    scale = case.scale if scale is None else scale
    _say(f"[fwd] {case.name} causal={case.causal} seed={case.seed} scale={scale}")
    qb, kb, vb = si.fwd_inputs(case)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o, lse = fa.fwd(q, k, v, causal=case.causal, scale=scale)
    import torch
    torch.cuda.synchronize()
    o_np, lse_np = to_f64(o), to_f64(lse)
    del q, k, v, o, lse
    qf, kf, vf = si.bf16_bits_to_f32(qb), si.bf16_bits_to_f32(kb), si.bf16_bits_to_f32(vb)
    if case.sampled_rows:
        # Forced rows first, then the seeded sample's other rows: the same count for every head.
        extra = np.unique(np.asarray(extra_rows, dtype=np.int64))
        assert len(extra) < case.sampled_rows
        rows = np.stack([np.sort(np.concatenate([
            extra, np.setdiff1d(si.sample_rows(case.seed, h, case.N, case.sampled_rows), extra)
                   [:case.sampled_rows - len(extra)]])) for h in range(case.Hq)])
    else:
        rows = None
    # One oracle pass over [V, |V|]: O and the P|V| term of the element bound.
    vx = np.concatenate([vf, np.abs(vf)], axis=-1)
    ox_ref, lse_ref = fa_oracle.attention_ref(qf, kf, vx, case.causal, scale, rows=rows)
    o_ref, pabs_ref = ox_ref[..., :case.d], ox_ref[..., case.d:]
    del vx, ox_ref
    if rows is not None:
        o_np = np.stack([o_np[:, h, rows[h]] for h in range(case.Hq)], axis=1)
        lse_np = np.stack([lse_np[:, h, rows[h]] for h in range(case.Hq)], axis=1)
    standard_scale = abs(scale - case.scale) < 1e-12
    stats = check_o(o_np, o_ref, pabs_ref, case.name, flat_gate=standard_scale, split=_may_split(case))
    stats["lse_rel"] = check_lse(lse_np, lse_ref, case.name)
    return stats


@pytest.mark.parametrize("case", [si.TINY, si.ONE_HEAD_8K, si.ONE_HEAD_8K_CAUSAL, si.HEADS32_4K,
                                  si.HEADS32_4K_CAUSAL], ids=lambda c: c.name)
def test_workloads(case):
    _run_case(case)


def test_long_context_128k_causal():
    _run_case(si.LONG_128K)


def test_causal_8k_many_heads():
    """8 heads of 8K causal: enough 256-row blocks to fill the CUs, so the
    8-wave kernel runs unsplit (the 1-head 8K causal case takes the split path)."""
    _run_case(si.FwdCase("1x8x8192 d128 causal", 1, 8, 8, 8192, 128, True, seed=41, sampled_rows=256))


@pytest.mark.parametrize("Hkv,d", [(32, 64), (8, 128)])
def test_causal_two_blocks_per_cu(Hkv, d):
    """32 causal heads of 4K: on a 256-CU part their 256-row blocks make exactly two per CU, which the
    BF16 planner runs as 8-wave blocks (heads interleaved per XCD, heaviest first); d = 64, and GQA."""
    _run_case(si.FwdCase(f"1x32x4096 d{d} causal kv{Hkv}", 1, 32, Hkv, 4096, d, True, seed=60 + d + Hkv,
                         sampled_rows=256))


@pytest.mark.parametrize("Hq,Hkv,N,d", [(16, 16, 8000, 128), (16, 4, 8000, 64), (8, 8, 8200, 128)])
def test_causal_eight_wave_ragged_tail(Hq, Hkv, N, d):
    """Causal shapes the planner runs as 256-row (8-wave) blocks with N not a multiple of 256: 16 heads
    of 8000 keys make exactly two blocks per CU, 8 heads of 8200 run unsplit. The last block is partial
    (staged Q rows clamped, the diagonal mask and rows past N together); every row of its tail, the
    rows at N - 256 and the first row of that block are checked beside the seeded sample."""
    last0 = (N - 1) // 256 * 256
    extra = sorted(set(range(last0, N)) | {N - 256, N - 255, last0 - 1})
    _run_case(si.FwdCase(f"1x{Hq}x{N} d{d} causal kv{Hkv} (8-wave ragged)", 1, Hq, Hkv, N, d, True,
                         seed=70 + Hq + d, sampled_rows=128), extra_rows=extra)


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 24, 24, 300, 64), (2, 8, 4, 500, 128), (1, 16, 2, 190, 128)])
def test_causal_head_groups(B, Hq, Hkv, N, d):
    """Causal grids whose B*Hq is a multiple of 8 (>= 16) interleave the blocks
    of B*Hq/8 heads in the grid order (groups of 3, 2 and 2 heads here)."""
    _run_case(si.FwdCase(f"head groups B{B} Hq{Hq} Hkv{Hkv} N{N} d{d}", B, Hq, Hkv, N, d, True,
                         seed=1300 + Hq + N))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_rescale_every_tile(d, causal):
    import torch
    import exact_tiled_attention_fa_amd as fa
    N = 640
    q, k, v = si.growing_score_inputs(N, d, seed=1500 + d)
    qb, kb, vb = si.bf16_round_bits(q), si.bf16_round_bits(k), si.bf16_round_bits(v)
    scale = 1.0 / math.sqrt(d)
    _say(f"[fwd] growing scores N{N} d{d} causal={causal}")
    o, lse = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = to_f64(o), to_f64(lse)
    qf, kf, vf = si.bf16_bits_to_f32(qb), si.bf16_bits_to_f32(kb), si.bf16_bits_to_f32(vb)
    vx = np.concatenate([vf, np.abs(vf)], axis=-1)
    ox_ref, lse_ref = fa_oracle.attention_ref(qf, kf, vx, causal, scale)
    o_ref, pabs_ref = ox_ref[..., :d], ox_ref[..., d:]
    # The last key of each row dominates; still, every tile raised the max.
    s_last = qf[0, 0, :, 0].astype(np.float64) * kf[0, 0, -1, 0] * scale * math.log2(math.e)
    assert s_last.min() > 8 * (N // 64)
    split = fa.fwd_workspace_bytes(1, 2, N, d) > 0
    check_o(o_np, o_ref, pabs_ref, f"growing N{N} d{d}", flat_gate=False, split=split)
    check_lse(lse_np, lse_ref, f"growing N{N} d{d}")


@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(N, d, causal):
    case = si.FwdCase(f"ragged N{N} d{d}", 2, 4, 2, N, d, causal, seed=1000 + N + d)
    _run_case(case)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.5])
def test_scale_edge_cases(scale):
    for causal in (False, True):
        case = si.FwdCase(f"scale {scale}", 1, 2, 1, 300, 128, causal, seed=77)
        _run_case(case, scale=scale)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (4, 4), (8, 1)])
def test_gqa_mapping(Hq, Hkv):
    _run_case(si.FwdCase(f"gqa {Hq}/{Hkv}", 2, Hq, Hkv, 256, 64, True, seed=50 + Hq + Hkv))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_query(causal, d):
    """One KV head for 32 query heads, two sequences: every query head of a sequence reads the same
    K and V."""
    _run_case(si.FwdCase(f"mqa 32/1 d{d}", 2, 32, 1, 300, d, causal, seed=55 + d + int(causal)))


def test_run_to_run_bitwise_determinism():
    import torch
    import exact_tiled_attention_fa_amd as fa
    case = si.FwdCase("determinism", 1, 8, 8, 2048, 128, False, seed=9)
    q, k, v = (to_dev(x) for x in si.fwd_inputs(case))
    o1, l1 = fa.fwd(q, k, v, causal=False)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    o3, l3 = fa.fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1, l3)
    assert not torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_fwd_on_concurrent_streams():
    """fa_fwd on the key-split path takes its partial buffer from the stream-ordered pool of the call's
    stream. Two streams, each running several calls back to back on its own inputs (both masks) with no
    synchronisation between them, must each get exactly fa_fwd_ws's results."""
    import torch
    import exact_tiled_attention_fa_amd as fa
    cases = [si.FwdCase("streams a", 1, 1, 1, 8192, 128, False, seed=91),
             si.FwdCase("streams b", 1, 2, 1, 6000, 128, True, seed=92)]
    assert all(fa.fwd_workspace_bytes(c.B, c.Hq, c.N, c.d) > 0 for c in cases)  # both take the split path
    inputs = [tuple(to_dev(x) for x in si.fwd_inputs(c)) for c in cases]
    refs = []
    for c, (q, k, v) in zip(cases, inputs):
        o = torch.empty_like(q)
        lse = torch.empty((c.B, c.Hq, c.N), dtype=torch.float32, device=q.device)
        fa.prepare_fwd(q, k, v, o, lse, causal=c.causal)()
        refs.append((o, lse))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for rep in range(4):
        for i, (c, (q, k, v)) in enumerate(zip(cases, inputs)):
            with torch.cuda.stream(streams[i]):
                outs[i].append(fa.fwd(q, k, v, causal=c.causal))
    torch.cuda.synchronize()
    for i, (o_ref, l_ref) in enumerate(refs):
        for o, lse in outs[i]:
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{cases[i].name}: O differs"
            assert torch.equal(lse, l_ref), f"{cases[i].name}: lse differs"


@pytest.mark.parametrize("shape", [(1, 1, 8192, 128, False), (1, 2, 6000, 128, True), (2, 32, 2048, 64, False)],
                         ids=["split", "split-causal", "single"])
def test_fwd_ws_timed_matches_fwd_ws(shape):
    """fa_fwd_ws_timed (the bench's way to time the attention kernel alone) gives fa_fwd_ws's results bit
    for bit, and records its event between the call's start and end: before the merge on the key-split
    path, at the end of the single launch otherwise."""
    import torch
    import exact_tiled_attention_fa_amd as fa
    B, H, N, d, causal = shape
    case = si.FwdCase("timed", B, H, H, N, d, causal, seed=97)
    print(f"[timed] B{B} H{H} N{N} d{d} causal={causal}", flush=True)
    q, k, v = (to_dev(x) for x in si.fwd_inputs(case))
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    l2 = torch.empty_like(l1)
    fa.prepare_fwd(q, k, v, o1, l1, causal=causal)()
    run = fa.prepare_fwd(q, k, v, o2, l2, causal=causal)
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    for rep in range(3):
        o2.fill_(float("nan"))
        start.record()
        run(after_attention=mid)
        end.record()
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), o1.view(torch.int16)), f"rep {rep}: O differs"
        assert torch.equal(l2, l1), f"rep {rep}: lse differs"
        t_mid, t_end = start.elapsed_time(mid), start.elapsed_time(end)
        assert 0.0 < t_mid <= t_end, (t_mid, t_end)


def test_equal_keys_give_mean_of_values_at_full_size():
    """Property at the 8K size: identical keys make every weight 1/N (causal: 1/(i+1))."""
    import torch
    import exact_tiled_attention_fa_amd as fa
    N, d = 8192, 128
    rng = np.random.default_rng(31)
    qb = si.normal_bf16(rng, (1, 1, N, d))
    krow = si.normal_bf16(rng, (d,))
    kb = np.broadcast_to(krow, (1, 1, N, d)).copy()
    vb = si.normal_bf16(rng, (1, 1, N, d))
    o, lse = fa.fwd(to_dev(qb), to_dev(kb), to_dev(vb), causal=True, scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    vf = si.bf16_bits_to_f32(vb)[0, 0].astype(np.float64)
    prefix_mean = np.cumsum(vf, 0) / np.arange(1, N + 1)[:, None]
    prefix_abs = np.cumsum(np.abs(vf), 0) / np.arange(1, N + 1)[:, None]
    check_o(to_f64(o)[0, 0], prefix_mean, prefix_abs, "equal keys causal", split=True)
    s = (si.bf16_bits_to_f32(qb)[0, 0].astype(np.float64) @ si.bf16_bits_to_f32(krow).astype(np.float64)) / math.sqrt(d)
    check_lse(to_f64(lse)[0, 0], s + np.log(np.arange(1, N + 1)), "equal keys causal lse")


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 1, 1, 8192, 64), (1, 1, 1, 16384, 128), (2, 1, 1, 12000, 128),
                                         (1, 2, 1, 4096, 128), (1, 3, 3, 3000, 64), (1, 8, 2, 2048, 128),
                                         (1, 1, 1, 8200, 128), (1, 2, 2, 9001, 64)])
def test_causal_split_per_block(B, Hq, Hkv, N, d):
    """Causal grids too small for the CUs split each block's keys by its own visible tiles (the heavy
    blocks into more splits, blocks that fit one split written directly); ragged N, GQA and d = 64 too."""
    rows = 256 if N > 4096 else None
    extra = [N - 1, N - 2, N - 64, N - 65] if rows else ()
    _run_case(si.FwdCase(f"causal split B{B} Hq{Hq} Hkv{Hkv} N{N} d{d}", B, Hq, Hkv, N, d, True,
                         seed=1700 + N + d + Hq, sampled_rows=rows), extra_rows=extra)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 1, 4096, 128, False), (1, 2, 3000, 64, True),
                                            (1, 1, 1100, 128, True), (2, 1, 2500, 128, False)])
def test_key_split_path(B, H, N, d, causal):
    """Grids of a few dozen work-groups take the key-split path (partials + combine)."""
    _run_case(si.FwdCase(f"split B{B} H{H} N{N} d{d}", B, H, H, N, d, causal, seed=600 + N + d))
