"""Pins of the speculative-sampling oracle (CPU): a hand-worked example,
closed cases, a brute-force inverse CDF and the law of speculative sampling
(the first emitted token is distributed as the target distribution)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_example():
    with open(os.path.join(GOLDEN, "spec_sampling.json")) as f:
        g = json.load(f)
    out, acc = oracle.chain_speculative_sampling(
        np.array(g["draft_probs"]), np.array(g["draft_token_ids"]), np.array(g["target_probs"]),
        np.array(g["accept_u"]), np.array(g["sample_u"]))
    assert out.tolist() == g["output_token_ids"]
    assert acc.tolist() == g["num_accepted"]


def test_inverse_cdf_matches_a_loop():
    rng = np.random.default_rng(81)
    for _ in range(200):
        V = int(rng.integers(1, 40))
        w = (rng.random(V) * (rng.random(V) < 0.6)).astype(np.float32)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        s = float(rng.random())
        total = 0.0
        for x in w:
            total += float(x)
        thr = float(np.float32(s)) * total
        run = 0.0
        want = None
        for k, x in enumerate(w):
            run += float(x)
            if run > thr:
                want = k
                break
        if want is None:
            want = max(k for k in range(V) if w[k] > 0)
        assert oracle.inverse_cdf(w, s) == want
    # a uniform that rounding pushes past the total lands on the last positive weight
    assert oracle.inverse_cdf(np.array([0.5, 0.5, 0.0], np.float32), 0.99999999) == 1


def test_identical_draft_accepts_everything():
    rng = np.random.default_rng(82)
    B, n, V = 6, 4, 50
    q = rng.random((B, n + 1, V)).astype(np.float32)
    q /= q.sum(axis=2, keepdims=True)
    ids = rng.integers(0, V, size=(B, n))
    out, acc = oracle.chain_speculative_sampling(q[:, :n], ids, q, rng.random((B, n)),
                                                 rng.random(B))
    assert (acc == n).all() and (out[:, :n] == ids).all() and (out[:, n] >= 0).all()


def test_disjoint_support_rejects_first_and_draws_from_target():
    rng = np.random.default_rng(83)
    B, n, V = 5, 3, 10
    q = np.zeros((B, n, V), np.float32)
    q[:, :, :5] = 0.2
    p = np.zeros((B, n + 1, V), np.float32)
    p[:, :, 5:] = rng.random((B, n + 1, 5)).astype(np.float32)
    p /= p.sum(axis=2, keepdims=True)
    ids = rng.integers(0, 5, size=(B, n))
    s = rng.random(B)
    out, acc = oracle.chain_speculative_sampling(q, ids, p, rng.random((B, n)), s)
    assert (acc == 0).all() and (out[:, 1:] == -1).all()
    for b in range(B):
        assert out[b, 0] == oracle.inverse_cdf(p[b, 0], s[b]) and out[b, 0] >= 5


def test_first_token_follows_the_target_distribution():
    """Speculative sampling is exact: whatever the draft distribution, the first
    emitted token is distributed as p_0 (Monte Carlo, 30000 draws)."""
    rng = np.random.default_rng(84)
    V, n, B = 5, 2, 30000
    p0 = np.array([0.05, 0.4, 0.15, 0.3, 0.1], np.float32)
    q0 = np.array([0.3, 0.1, 0.3, 0.1, 0.2], np.float32)
    p = np.broadcast_to(np.stack([p0, p0, p0]), (B, n + 1, V))
    q = np.broadcast_to(np.stack([q0, q0]), (B, n, V))
    q64 = q0.astype(np.float64) / q0.astype(np.float64).sum()
    ids = np.stack([rng.choice(V, size=B, p=q64) for _ in range(n)], 1)
    out, acc = oracle.chain_speculative_sampling(q, ids, p, rng.random((B, n)), rng.random(B))
    freq = np.bincount(out[:, 0], minlength=V) / B
    assert np.abs(freq - p0).max() < 0.012
    # and the acceptance rate of the first draft is sum_x min(p, q)
    assert abs((acc >= 1).mean() - np.minimum(p0, q0).sum()) < 0.012
