"""Host logic of bench.py: the algorithmic bytes and FLOPs each kernel class is
judged by (written out here from the shapes of the 30-layer canvas loop), the
roofline arithmetic, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_c2_moe_and_lm_head():
    cfg = get_config("c2")
    T, d, E, k, de, V = 256, 2048, 128, 8, 704, 262144
    b, f = bench.algorithmic(cfg, "moe_gateup")
    # every expert's gate and up rows once, the normed tokens in, h out
    assert b == E * 2 * de * d * 2 + T * d * 2 + T * k * de * 2 == 742_129_664
    assert f == 2.0 * T * k * 2 * de * d
    b, f = bench.algorithmic(cfg, "moe_down")
    assert b == E * d * de * 2 + T * k * de * 2 + T * k * d * 4
    assert round(b / 1e6, 1) == 388.8
    b, f = bench.algorithmic(cfg, "lm_head")
    assert b == V * d * 2 + T * d * 2
    assert round(f / 1e9, 1) == 274.9  # 2 T V d


def test_algorithmic_c2_dense_and_attention():
    cfg = get_config("c2")
    T, d, A, keys = 256, 2048, 16 * 128, 2048 + 256
    b, f = bench.algorithmic(cfg, "qkv")
    assert b == 3 * A * d * 2 + T * d * 2 + 3 * T * A * 2 and round(b / 1e6, 1) == 29.4
    assert f == 2.0 * T * 3 * A * d
    b, f = bench.algorithmic(cfg, "attn")
    assert b == keys * A * 2 * 2 + 2 * T * A * 2
    assert f == 4.0 * T * keys * A


def test_router_logits_follow_the_launch_that_computes_them():
    c2, c3, c4 = get_config("c2"), get_config("c3"), get_config("c4")
    assert bench.router_in_shared(c2)          # bf16, 256 tokens
    assert not bench.router_in_shared(c3)      # 1024 pooled tokens
    assert not bench.router_in_shared(c4)      # fp8 shared expert
    T, d, E, ds = 256, 2048, 128, 2048
    logits = E * d * 2 + T * E * 4, 2.0 * T * E * d
    # c2: the top-k rides in the shared down launch too, so its bytes join the shared class
    assert bench.topk_in_shared(c2) and not bench.topk_in_shared(c3) and not bench.topk_in_shared(c4)
    topk = T * E * 4 + 2 * T * 8 * 4
    sb, sf = bench.algorithmic(c2, "shared")
    base_b = 3 * ds * d * 2 + T * d * 2 + 2 * T * ds * 2 + T * d * 4
    assert (sb, sf) == (base_b + topk + logits[0], 2.0 * T * 3 * ds * d + logits[1])
    rb, rf = bench.algorithmic(c2, "router")
    assert (rb, rf) == (topk, 0.0)
    # batch 4: the router GEMM is its own launch and its bytes stay in the router class
    T4 = 1024
    rb, rf = bench.algorithmic(c3, "router")
    assert rb == T4 * E * 4 + 2 * T4 * 8 * 4 + E * d * 2 + T4 * E * 4 + T4 * d * 2
    assert rf == 2.0 * T4 * E * d


def test_fp8_experts_count_codes_and_row_scales():
    cfg = get_config("c4")
    E, d, de = 128, 2048, 704
    b, _ = bench.algorithmic(cfg, "moe_gateup")
    assert b == E * 2 * de * d + E * 2 * de * 4 + 256 * d * 2 + 256 * 8 * de * 2


def test_mxfp4_experts_count_codes_and_block_scales():
    """Half a byte per weight plus one E8M0 byte per 32 weights; the shared
    expert stays bf16."""
    cfg = get_config("c6")
    E, d, de, T, k = 128, 2048, 704, 256, 8
    b, f = bench.algorithmic(cfg, "moe_gateup")
    assert b == E * 2 * de * d // 2 + E * 2 * de * d // 32 + T * d * 2 + T * k * de * 2
    assert f == 2.0 * T * k * 2 * de * d
    b, _ = bench.algorithmic(cfg, "moe_down")
    assert b == E * d * de // 2 + E * d * de // 32 + T * k * de * 2 + T * k * d * 4
    sb, _ = bench.algorithmic(cfg, "shared")
    assert sb == bench.algorithmic(get_config("c2"), "shared")[0]


def test_roofline_entry_arithmetic():
    cfg = get_config("c2")
    b, _ = bench.algorithmic(cfg, "moe_gateup")
    e = bench.roofline_entry(cfg, "moe_gateup", total_ms=117.6 * 1440 / 1000, launches=1440)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0
    assert e["avg_launch_us"] == pytest.approx(117.6)
    assert e["achieved"] == pytest.approx(b / 117.6e-6 / 1e9)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0)
    _, f = bench.algorithmic(cfg, "lm_head")
    e = bench.roofline_entry(cfg, "lm_head", total_ms=0.330 * 48, launches=48)
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s" and e["peak"] == 2500.0
    assert e["achieved"] == pytest.approx(f / 330e-6 / 1e12)


def test_measured_traffic_is_near_the_algorithmic_bytes():
    cfg = get_config("c2")
    b, _ = bench.algorithmic(cfg, "moe_gateup")
    t = bench.MEASURED_TRAFFIC[("moe_gateup", cfg.name)]
    assert b <= t <= 1.05 * b


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, cwd=ROOT,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
