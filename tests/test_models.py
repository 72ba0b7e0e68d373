"""Pins for the analytic byte/FLOP models against every number the pages print."""
import os

import pytest

from oracle import fa_models as fm

MiB = fm.MiB


def _kv(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            parts = line.split()
            out[parts[0]] = parts[1:]
    return out


def _rows(path):
    return [line.split() for line in open(path) if line.strip() and not line.startswith("#")]


def test_p1_one_head_8k(golden_dir):
    """"FlashAttention HBM bytes, one head, 8K": every printed count."""
    g = _kv(os.path.join(golden_dir, "p1_hbm_bytes.txt"))

    def val(name):
        return float(g[name][0]), int(g[name][2])

    N, d = int(val("N")[0]), int(val("d")[0])
    bw = val("h100_bw_tbs")[0] * 1e12
    peak = val("h100_peak_tflops")[0] * 1e12

    def check(name, x):
        v, dec = val(name)
        assert round(x, dec) == v, (name, x, v)

    check("tensor_mib", fm.tensor_bytes(N, d) / MiB)
    check("compulsory_mib", fm.compulsory_bytes(N, d) / MiB)
    check("score_matrix_mib", N * N * 2 / MiB)
    check("score_traffic_mib", (fm.naive_bytes(N, d) - fm.compulsory_bytes(N, d)) / MiB)
    check("naive_total_mib", fm.naive_bytes(N, d) / MiB)
    check("naive_total_1e6_bytes", fm.naive_bytes(N, d) / 1e6)
    check("naive_time_us", fm.naive_bytes(N, d) / bw * 1e6)
    check("paper_model_br128_blocks", N // 128)
    check("paper_model_br128_kv_mib", (fm.paper_model_bytes(N, d, 128) - 2 * fm.tensor_bytes(N, d)) / MiB)
    check("paper_model_br128_total_mib", fm.paper_model_bytes(N, d, 128) / MiB)
    check("paper_model_br64_total_mib", fm.paper_model_bytes(N, d, 64) / MiB)
    check("real_hbm_1e6_bytes", fm.compulsory_bytes(N, d) / 1e6)
    check("fwd_gflop", fm.fwd_flops(N, d) / 1e9)
    check("intensity_flop_per_byte", fm.fwd_flops(N, d) / fm.compulsory_bytes(N, d))
    check("h100_ridge_flop_per_byte", peak / bw)
    check("compute_time_us", fm.fwd_flops(N, d) / peak * 1e6)
    check("hbm_time_us", fm.compulsory_bytes(N, d) / bw * 1e6)
    check("naive_over_real", fm.naive_bytes(N, d) / fm.compulsory_bytes(N, d))
    check("causal_gflop", fm.fwd_flops(N, d, causal=True) / 1e9)
    check("decode_kv_mib_per_kv_head", fm.decode_kv_bytes(N, d) / MiB)
    check("decode_flop_per_byte_per_group_member", fm.decode_intensity(N, d, group=1))
    assert fm.decode_intensity(N, d, group=4) == 4.0
    # FP32 scores double the naive score traffic.
    assert fm.naive_bytes(N, d, score_elem=4) - fm.compulsory_bytes(N, d) == \
        2 * (fm.naive_bytes(N, d) - fm.compulsory_bytes(N, d))


def test_p2_footprint_table(golden_dir):
    for n, std, fl, red, sav in _rows(os.path.join(golden_dir, "p2_footprint_table.txt")):
        n = int(n)
        s = fm.standard_footprint_gib(n, 32, 128)["total"] * 1024
        f = fm.flash_footprint_gib(n, 32, 128)["total"] * 1024
        assert round(s, 1) == float(std)
        assert round(f, 1) == float(fl)
        assert round(s / f, 1) == float(red)
        assert round(s - f, 1) == float(sav)


def test_p2_score_table(golden_dir):
    for n, gb in _rows(os.path.join(golden_dir, "p2_score_table.txt")):
        assert round(fm.standard_footprint_gib(int(n), 32, 128)["scores"], 2) == float(gb)


def test_p2_traffic_table(golden_dir):
    for n, std, fl, red in _rows(os.path.join(golden_dir, "p2_traffic_table.txt")):
        t = fm.hbm_traffic_gib(int(n), 32, 128)
        assert round(t["standard"], 2) == float(std)
        assert round(t["flash"], 3) == float(fl)
        assert round(t["reduction"], 1) == float(red)


def test_p2_sram_table(golden_dir):
    for row in _rows(os.path.join(golden_dir, "p2_sram_table.txt")):
        if row[0] == "best":
            budget, block, ai = float(row[1]), int(row[2]), float(row[3])
            assert fm.best_block(budget, 128) == block
            assert fm.tile_intensity(block, 128) == ai
            continue
        b = int(row[0])
        u = fm.sram_usage_kib(b, 128)
        assert round(u["q"], 1) == float(row[1])
        assert round(u["kv"], 1) == float(row[2])
        assert round(u["out"], 1) == float(row[3])
        assert round(u["stats"], 1) == float(row[4])
        assert round(u["total"], 1) == float(row[5])
        assert (u["total"] <= 192) == (row[6] == "YES")
        assert fm.tile_intensity(b, 128) == float(row[7])


def test_p3_traffic(golden_dir):
    g = _kv(os.path.join(golden_dir, "p3_traffic.txt"))

    def check(name, x):
        v, dec = float(g[name][0]), int(g[name][1])
        assert round(x, dec) == v, (name, x, v)

    d, flops, bw = 64, 300e12, 2e12
    check("score_entries_4096", 4096 * 4096)
    check("score_mib_per_head_4096", 4096 * 4096 * 2 / MiB)
    check("machine_balance", fm.machine_balance(flops, bw))
    check("softmax_flop_per_byte", 5 / 4)
    check("standard_mb_4096", fm.standard_traffic_bytes(4096, d) / 1e6)
    check("standard_mb_8192", fm.standard_traffic_bytes(8192, d) / 1e6)
    check("four_pass_mb_4096", 4 * 4096 * 4096 * 2 / 1e6)
    bc = fm.tiled_kv_block(int(g["sram_numbers"][0]), d)
    check("block_cols", bc)
    check("passes_4096", 4096 // bc)
    check("tiled_mb_4096", fm.tiled_traffic_bytes(4096, d, bc) / 1e6)
    check("tiled_mb_8192", fm.tiled_traffic_bytes(8192, d, bc) / 1e6)
    check("reduction_4096", fm.standard_traffic_bytes(4096, d) / fm.tiled_traffic_bytes(4096, d, bc))
    check("standard_time_us_4096", fm.standard_traffic_bytes(4096, d) / bw * 1e6)
    check("arithmetic_time_us_4096", fm.fwd_flops(4096, d) / flops * 1e6)
    check("tiled_time_us_4096", fm.tiled_traffic_bytes(4096, d, bc) / bw * 1e6)


@pytest.mark.parametrize("N,expect_mib", [(8192, 8), (4096, 4)])
def test_compulsory_floor_scales_linearly(N, expect_mib):
    assert fm.compulsory_bytes(N, 128) == expect_mib * MiB
