"""The seeded input generator: shapes, storage rounding and determinism."""
import json
import os

import numpy as np
import torch

from sparse_attention_diffusion_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_case_figures_match_its_definition():
    with open(os.path.join(GOLDEN, "workload_figures.json")) as f:
        fig = json.load(f)["tiny_case"]
    wl = W.WORKLOADS["tiny"]
    assert wl.n == fig["n"] and wl.group == fig["group"]
    assert wl.groups == fig["groups"]
    assert wl.topk(fig["density"]) == fig["topk"]


def test_grid_token_order_is_row_major():
    c = W.grid_coords((2, 3, 4))
    assert c.shape == (24, 3)
    t, y, x = 1, 2, 3
    assert (c[(t * 3 + y) * 4 + x] == [t, y, x]).all()


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -2.00390625, 0.0]  # exact ties
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert (W.round_bf16(x) == want).all()


def test_generator_is_deterministic_and_drifts():
    wl = W.WORKLOADS["tiny"]
    a = W.make_qkv(wl)
    b = W.make_qkv(wl)
    for x, y in zip(a, b):
        assert (x == y).all()
    c = W.make_qkv(wl, step=1)
    dq = (c[0] - a[0]).std()
    assert 0.03 < dq < 0.07  # one random-walk step of sigma 0.05


def test_feature_statistics():
    wl = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(wl)
    assert q.shape == (1, 1024, 64) and q.dtype == np.float32
    # unit-variance features plus 0.5^2 noise
    assert abs(q.var() - 1.25) < 0.1 and abs(v.var() - 1.0) < 0.05


def test_pct_of_ideal_reproduces_the_pages_kernel_speed_figure():
    # summary page, kernel-speed paragraph: 4.79x at density 0.2 is 96% of the
    # ideal 1/density speedup; bench.py reports its own ratio the same way
    import bench
    with open(os.path.join(GOLDEN, "workload_figures.json")) as f:
        fig = json.load(f)["kernel_speed"]
    got = bench.pct_of_ideal(fig["speedup_vs_fa3"], fig["density"])
    assert abs(got - 0.958) < 1e-12
    assert round(got, 2) == fig["fraction_of_ideal"]
    assert W.WORKLOADS["wan14b_720p"].n == fig["tokens"]


def test_schedule_cost_closed_forms():
    # the trajectory's own schedule (5 dense steps, anchors every 5 of 50) with unit
    # dense cost, anchor = 2 and reuse = density: 5 + 9 * 2 + 36 * 0.15 = 28.4
    from sparse_attention_diffusion_amd.drift import schedule_cost
    sp, ov = schedule_cost(1.0, 2.0, 0.15, 50, 5, 5, 0.15)
    assert abs(sp - 50 / 28.4) < 1e-12
    assert abs(ov - (28.4 - 5 - 45 * 0.15) / 45 * 100) < 1e-9
    # an anchor that costs no more than a reuse step adds nothing over the density
    sp, ov = schedule_cost(1.0, 0.2, 0.2, 50, 0, 7, 0.2)
    assert abs(ov) < 1e-9 and abs(sp - 5.0) < 1e-12
    # gap 1: every sparse step is an anchor
    sp, ov = schedule_cost(1.0, 3.0, 0.1, 10, 2, 1, 0.1)
    assert abs(sp - 10 / (2 + 8 * 3.0)) < 1e-12
