"""The seeded input generator: determinism, regeneration of single units and
position ranges, bf16 rounding, and the budget integers of the workloads."""
import json
import os

import numpy as np
import pytest
import torch

from workload import WORKLOADS, budget_from_percent, get, scaled, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_budget_integers_match_printed_values():
    with open(os.path.join(GOLDEN, "budgets.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert budget_from_percent(c["percent"], c["prompt_len"]) == c["heavy"]
        assert 2 * budget_from_percent(c["percent"], c["prompt_len"]) == c["k"]


def test_workload_budgets():
    assert get("tiny-fp32").k == 52
    assert (get("opt6.7b-layer-b16").heavy_budget, get("opt6.7b-layer-b16").recent_budget) == (52, 52)
    assert get("opt6.7b-32L-b64").heavy_budget == 205
    assert [get(f"opt30b-b128-{p}pct").heavy_budget for p in (4, 10, 20, 100)] == [21, 52, 103, 1024]
    full = get("opt30b-b128-100pct")
    assert full.k >= full.n_positions  # the 100% run never evicts
    assert get("llama7b-stream-4m").k == 2048


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.00390625, 3.0e-39, 0.0, -0.0], np.float32)])
    ours = synth.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    t = synth.to_torch(get("opt6.7b-layer-b16"), ours)
    assert torch.equal(t.to(torch.float32), torch.from_numpy(ours))


def test_unit_regeneration_and_ranges():
    w = scaled(get("opt6.7b-layer-b16"), batch=2, heads=3, prompt_len=900, decode_steps=300)
    Q, K, V = synth.batch_qkv(w, 0)
    q, k, v = synth.unit_qkv(w, 0, 1, 2)
    assert np.array_equal(q, Q[1, 2]) and np.array_equal(k, K[1, 2]) and np.array_equal(v, V[1, 2])
    q2, k2, v2 = synth.unit_qkv(w, 0, 1, 2, start=1000, stop=1100)  # crosses a chunk boundary
    assert np.array_equal(k2, K[1, 2, 1000:1100]) and np.array_equal(q2, Q[1, 2, 1000:1100])
    # values are exactly bf16
    assert np.array_equal(synth.round_to_bf16(K), K)
    # another layer or head draws different values
    assert not np.array_equal(synth.unit_qkv(w, 1, 1, 2)[1], k)


def test_anchor_layouts():
    w = get("opt6.7b-layer-b16")
    alpha, ke, qe = synth.anchors(w, 0, 0)
    assert (alpha > 0).sum() == w.n_anchors == 11
    assert set(np.unique(alpha)) == {0.0, np.float32(3.0)}
    z = get("opt30b-b128-20pct")
    alpha, _, _ = synth.anchors(z, 0, 3)
    assert alpha.max() == pytest.approx(3.0) and alpha.min() == pytest.approx(3.0 * 2048 ** -1.1, rel=1e-6)
    s = scaled(get("llama7b-stream-4m"), decode_steps=50_000)
    alpha, ke, qe = synth.anchors(s, 0, 0)
    assert (alpha > 0).sum() == s.n_anchors + 5
    assert np.all(np.diff(qe) >= 0) and qe[-1] == 5
    # a query's epoch is the latest key anchor at or before it
    starts = np.nonzero(ke)[0]
    assert qe[starts[2]] == 3 and qe[starts[2] - 1] == 2
    u0, u1 = synth.direction(s, 0, 0, 0), synth.direction(s, 0, 0, 1)
    assert abs(np.linalg.norm(u0) - 1) < 1e-6 and abs(u0 @ u1) < 0.5


def test_query_bias_direction():
    w = scaled(get("opt6.7b-layer-b16"), batch=1, heads=2, prompt_len=512, decode_steps=512)
    Q, K, _ = synth.batch_qkv(w, 0)
    u = synth.direction(w, 0, 1)
    # queries carry +u: their mean projection on u is about 1; keys' about alpha * share of anchors
    assert abs(Q[0, 1] @ u).mean() > 0.5 and abs((Q[0, 1] @ u).mean() - 1.0) < 0.15


def test_torch_generator_deterministic():
    w = scaled(get("opt6.7b-32L-b64"), batch=2, heads=2, prompt_len=64, decode_steps=32)
    a = synth.torch_qkv(w, 3, 0, 96, "cpu")
    b = synth.torch_qkv(w, 3, 0, 96, "cpu")
    c = synth.torch_qkv(w, 3, 40, 96, "cpu")
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.equal(a[1][:, :, 40:], c[1])
    assert a[0].dtype == torch.bfloat16 and a[0].shape == (2, 2, 96, 128)
