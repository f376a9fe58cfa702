"""Seeded input generators: determinism, shapes and the stated distributions."""
import numpy as np
import pytest
import torch

from shared_history_candidate_amd import workloads as W


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.0, 0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(W.round_bf16(x), ref)


@pytest.mark.parametrize("name", ["tiny", "rest", "ragged"])
def test_deterministic(name):
    a, b = W.make(name, 0), W.make(name, 0)
    for f in ("cu_kv", "cu_cand", "Z", "wt", "K"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = W.make(name, 1)
    assert not np.array_equal(a.K[:16], c.K[:16])


def test_config_shapes():
    t = W.make("tiny")
    assert (t.R, t.q, t.d, t.heads, t.d_h, t.dtype) == (1, 3, 64, 2, 32, "fp32")
    assert t.total_kv == 64 and t.total_cand == 4 and t.V is None
    r = W.make("rest")
    assert (r.R, r.q, r.d, r.heads, r.total_cand) == (8, 3, 256, 4, 2048)
    assert r.lengths.min() >= 512 and r.lengths.max() <= 1024
    x = W.make("ragged")
    assert (x.R, x.q, x.d, x.heads, x.d_h) == (64, 3, 256, 8, 32)
    assert x.lengths.min() >= 256 and x.lengths.max() <= 4096
    assert x.cands.min() >= 1 and x.cands.max() <= 64


def test_bf16_values_are_representable():
    r = W.make("rest")
    for a in (r.Z, r.wt, r.K):
        assert np.array_equal(W.round_bf16(a), a)


def test_weight_variance():
    r = W.make("rest")
    assert abs(r.wt.var() - 1.0 / 256) < 0.05 / 256
    assert abs(r.K.var() - 1.0) < 0.02


def test_flops_and_bytes():
    t = W.make("tiny")
    m = 12
    assert t.flops() == 2 * m * 64 * 64 + 4 * m * 64 * 64
    assert t.bytes() == 4 * (64 * 64 + 2 * m * 64 + 3 * 64 * 64)
