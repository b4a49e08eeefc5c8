"""bench.py's host side: the one-GPU rule and the work it counts per step."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from gemv_skinny_gemm_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_step_work_of_a_dense_layer():
    # The TP=8 shard of one Qwen2.5-72B layer: QKV, O, gate_up, down.
    shapes = [(1280, 8192), (8192, 1024), (7392, 8192), (8192, 3696)]
    specs = wl.tp8_layer(wl.BF16)
    assert [(s.N, s.K) for s in specs] == shapes
    flops, wbytes = bench.step_work(specs, 3)
    assert flops == 2 * 3 * sum(n * k for n, k in shapes)
    assert wbytes == 2 * sum(n * k for n, k in shapes)


def test_step_work_counts_fp8_scales():
    specs = wl.tp8_layer(wl.FP8_BS128)
    _, wbytes = bench.step_work(specs, 1)
    blocks = sum(-(-s.N // 128) * -(-s.K // 128) for s in specs)
    assert wbytes == sum(s.N * s.K for s in specs) + 4 * blocks


def test_step_work_of_a_moe_step_counts_routes_and_chosen_experts():
    E, H, I = wl.MOE_EXPERTS, wl.MOE_HIDDEN, wl.MOE_INTER
    specs = wl.moe_experts(wl.FP8_BS128)
    # Three tokens, top 2: experts 0, 1, 5 chosen; one route to no expert.
    ids = np.array([[0, 1], [1, 5], [5, E]], dtype=np.int32)
    flops, wbytes = bench.step_work(specs, 3, ids)
    routes = 5
    assert flops == 2 * routes * (2 * I * H + H * I)
    per_expert = (2 * I * H + 4 * (2 * I // 128) * (H // 128)) + (H * I + 4 * (H // 128) * (I // 128))
    assert wbytes == 3 * per_expert
