"""The seeded generator: device-independent definition and the workloads' distributions."""
import math

import pytest

import numpy as np
import torch

import workload as w
from oracle import moe_oracle as oracle


def test_numpy_and_torch_hash_agree():
    for start in (0, 12345, (1 << 32) - 5000):
        a = w.uniform_bits(5000, 0xDEADBEEF, "cpu", start)
        b = w.uniform_bits_torch(5000, 0xDEADBEEF, "cpu", start)
        assert torch.equal(a, b)


def test_bits_look_uniform():
    b = w.uniform_bits(1 << 18, w.stream_key(0, 1), "cpu").numpy()
    for bit in (0, 5, 16, 24, 31):
        assert abs(((b >> bit) & 1).mean() - 0.5) < 0.01
    top = b >> 16
    counts = np.bincount(top % 64, minlength=64)
    assert counts.min() > 0.85 * counts.mean()


def test_streams_differ_and_are_reproducible():
    a = w.normal((64, 64), w.stream_key(0, w.T_X))
    b = w.normal((64, 64), w.stream_key(0, w.T_X))
    c = w.normal((64, 64), w.stream_key(1, w.T_X))
    assert torch.equal(a, b) and not torch.equal(a, c)
    # a slice regenerated with an element offset equals the slice of the whole tensor
    part = w.normal((16, 64), w.stream_key(0, w.T_X), start=32 * 64)
    assert torch.equal(part, a[32:48])


def test_normal_table_symmetric_with_std_002():
    t = w.normal_table().numpy().astype(np.float64)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.std() - 0.02) < 2e-4 and abs(t.mean()) < 1e-15
    x = w.normal((200000,), w.stream_key(3, 3)).numpy()
    assert abs(x.std() - 0.02) < 3e-4 and abs(x.mean()) < 3e-4


def test_router_logit_scale_matches_closed_form():
    cfg = w.CONFIGS["tiny_f32"].scaled(N=2048)
    x = w.hidden_states(cfg)
    w_r = w.router_weight(cfg)
    assert w_r.shape == (cfg.E, cfg.H) and w_r.dtype == x.dtype
    z = oracle.router_logits(x.double().numpy(), w_r.double().numpy())
    sigma = 0.02 * 0.02 * math.sqrt(cfg.H)
    assert abs(z.std() / sigma - 1) < 0.05


def test_zipf_bias_shape_and_order():
    cfg = w.CONFIGS["dsv3_zipf_bf16"]
    b = w.zipf_bias(cfg).numpy().astype(np.float64)
    assert b.shape == (256,)
    r = np.sort(b)[::-1]
    sigma = 0.02 * 0.02 * math.sqrt(cfg.H)
    # consecutive Zipf ranks differ by s * ln((r+1)/r) in units of sigma_z
    assert math.isclose(r[0] - r[1], sigma * 1.2 * math.log(2), rel_tol=1e-5)
    assert w.zipf_bias(w.CONFIGS["dsv3_bf16"]) is None


def test_fixed_routes_have_distinct_experts():
    for kind in ("round_robin", "hot", "random"):
        idx = w.fixed_route(300, 16, 5, kind).numpy()
        assert idx.shape == (300, 5) and idx.dtype == np.int32
        assert all(len(set(row)) == 5 for row in idx.tolist())


def test_batched_expert_generation_matches_per_expert_streams():
    cfg = w.CONFIGS["dsv3_bf16"].scaled(E=5, H=256, I=128)
    a13, a2 = w.all_expert_weights(cfg, "cpu")
    b13 = w._normal_streams([w.stream_key(cfg.seed, w.T_W13, e) for e in range(5)], (256, 256), "cpu",
                            torch.bfloat16)
    b2 = w._normal_streams([w.stream_key(cfg.seed, w.T_W2, e) for e in range(5)], (256, 128), "cpu",
                           torch.bfloat16)
    assert torch.equal(a13, b13) and torch.equal(a2, b2)


def test_counted_route_gives_the_requested_counts():
    n_e = [5, 0, 8, 3, 8, 8]
    idx = w.counted_route(n_e, 4, seed=3).numpy()
    assert idx.shape == (8, 4) and idx.dtype == np.int32
    assert all(len(set(row)) == 4 for row in idx.tolist())
    assert np.array_equal(np.bincount(idx.reshape(-1), minlength=6), n_e)
    with pytest.raises(ValueError):
        w.counted_route([10, 2], 2)        # 10 rows for one expert but only 6 tokens
    with pytest.raises(ValueError):
        w.counted_route([3, 2], 2)         # 5 slots are not a multiple of k
