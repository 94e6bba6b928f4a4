"""Pins of the sampling oracle (oracle/sampling.py) against closed forms,
invariants and an independent brute-force sampler.

* Greedy: temperature 0 gives the first index of the largest logit.
* top_k = 1 gives that same token at any temperature and draw.
* Equal logits: top_k = k keeps ids 0..k-1 (ties rank by id) and the draw u
  returns id floor(u * k) exactly.
* Two tokens with logits ln 3 and 0: token 0 iff u < 2^32 / (2^32 +
  floor(2^32 / 3)).
* Top-p on probabilities 0.5, 0.3, 0.15, 0.05 (shuffled ids): top_p = 0.5
  keeps the 0.5 token alone; 0.75 keeps it and the 0.3 token, drawn 5:3.
* A grid of draws reproduces the integer weights (each kept token's count
  is within one of N * q_i / R).
* Adding a constant to every logit (exactly representable values) changes
  nothing.
* Brute force: a separate sampler (sorted Python lists, fp64 probabilities,
  no integer weights) agrees on small random vocabularies wherever the draw
  is not within rounding of a boundary.
"""
import math

import numpy as np
import pytest

from oracle import sampling as S


def test_greedy_and_ties():
    lg = np.array([0.5, 2.0, -1.0, 2.0, 1.9], np.float32)
    for u in (0.0, 0.5, 0.999):
        assert S.sample(lg, 0.0, 0, 1.0, u).token == 1
        assert S.sample(lg, -1.0, 3, 0.5, u).token == 1


@pytest.mark.parametrize("T", [0.1, 0.7, 1.0, 5.0])
def test_top_k_one_is_argmax(T):
    rng = np.random.default_rng(3)
    for _ in range(20):
        lg = rng.normal(size=257).astype(np.float32)
        u = float(rng.random())
        assert S.sample(lg, T, 1, 1.0, u).token == int(np.argmax(lg))


@pytest.mark.parametrize("k", [1, 2, 7, 64, 100])
def test_equal_logits_closed_form(k):
    V = 100
    lg = np.full(V, 0.25, np.float32)
    for j in range(200):
        u = (j + 0.5) / 200
        d = S.sample(lg, 0.8, k, 1.0, u)
        assert d.token == math.floor(u * k), (k, u)
        assert d.kept.sum() == k and d.kept[:k].all()


def test_two_tokens_closed_form():
    lg = np.array([math.log(3.0), 0.0])
    q1 = math.floor(2.0 ** 32 / 3.0)
    u_star = 2.0 ** 32 / (2.0 ** 32 + q1)
    assert abs(u_star - 0.75) < 1e-9
    assert S.sample(lg, 1.0, 0, 1.0, u_star - 1e-7).token == 0
    assert S.sample(lg, 1.0, 0, 1.0, u_star + 1e-7).token == 1
    # temperature 2 flattens: weights 1 and 3^(-1/2)
    w1 = math.floor(3.0 ** -0.5 * 2.0 ** 32)
    u2 = 2.0 ** 32 / (2.0 ** 32 + w1)
    assert S.sample(lg, 2.0, 0, 1.0, u2 - 1e-7).token == 0
    assert S.sample(lg, 2.0, 0, 1.0, u2 + 1e-7).token == 1


def test_top_p_known_distribution():
    probs = {3: 0.5, 0: 0.3, 2: 0.15, 1: 0.05}  # token id -> probability
    lg = np.zeros(4)
    for t, p in probs.items():
        lg[t] = math.log(p)
    for j in range(100):
        u = (j + 0.5) / 100
        assert S.sample(lg, 1.0, 0, 0.5, u).token == 3
    # 0.75: tokens 3 and 0 remain (weights 1 and 0.6), drawn in id order
    counts = np.zeros(4, int)
    N = 1600
    for j in range(N):
        d = S.sample(lg, 1.0, 0, 0.75, (j + 0.5) / N)
        assert set(np.flatnonzero(d.kept)) == {0, 3}
        counts[d.token] += 1
    assert abs(counts[0] - N * 0.375) <= 1 and abs(counts[3] - N * 0.625) <= 1
    # top_k = 2 keeps the same two; top_k = 3 with top_p = 0.95 keeps three
    d = S.sample(lg, 1.0, 2, 1.0, 0.9)
    assert set(np.flatnonzero(d.kept)) == {0, 3}
    d = S.sample(lg, 1.0, 3, 0.95, 0.9)
    assert set(np.flatnonzero(d.kept)) == {0, 2, 3}


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.6, 20, 1.0), (1.3, 0, 0.8), (0.9, 50, 0.6)])
def test_grid_of_draws_matches_weights(T, k, p):
    rng = np.random.default_rng(11)
    lg = rng.normal(scale=2.0, size=300).astype(np.float32)
    N = 5000
    counts = np.zeros(lg.size, int)
    first = S.sample(lg, T, k, p, 0.5)
    for j in range(N):
        counts[S.sample(lg, T, k, p, (j + 0.5) / N).token] += 1
    R = first.q.sum()
    expect = N * first.q / R
    assert np.all(counts[~first.kept] == 0)
    assert np.all(np.abs(counts - expect) <= 1.0 + 1e-9)


def test_shift_invariance_exact_values():
    rng = np.random.default_rng(5)
    lg = rng.integers(-32, 33, size=500) / 8.0  # exact in fp32 and fp64
    for T, k, p in ((1.0, 0, 1.0), (0.5, 40, 0.9), (2.0, 0, 0.3)):
        for u in (0.01, 0.37, 0.999):
            a = S.sample(lg, T, k, p, u)
            b = S.sample(lg + 64.0, T, k, p, u)
            assert a.token == b.token and np.array_equal(a.kept, b.kept)


def _brute(lg, T, k, p, u):
    """Independent sampler: sorted Python lists, fp64 probabilities."""
    V = len(lg)
    ranked = sorted(range(V), key=lambda i: (-float(lg[i]), i))
    if not T > 0:
        return ranked[0]
    m = max(float(x) for x in lg)
    w = [math.exp((float(lg[i]) - m) / T) for i in range(V)]
    keep = ranked[:k] if 0 < k < V else ranked[:]
    if p < 1.0:
        tot = sum(w[i] for i in keep)
        acc, cut = 0.0, []
        for i in keep:
            cut.append(i)
            acc += w[i]
            if acc >= p * tot:
                break
        keep = cut
    keep = sorted(keep)
    tot = sum(w[i] for i in keep)
    acc = 0.0
    for i in keep:
        acc += w[i]
        if u * tot < acc:
            return i
    return keep[-1]


def test_brute_force_small_vocabularies():
    rng = np.random.default_rng(2024)
    checked = 0
    for case in range(3000):
        V = int(rng.integers(1, 12))
        lg = np.round(rng.normal(scale=1.5, size=V), 1)  # ties happen
        T = float(rng.choice([0.0, 0.3, 1.0, 2.5]))
        k = int(rng.integers(0, V + 2))
        p = float(rng.choice([1.0, 0.9, 0.6, 0.2]))
        u = float(rng.random())
        d = S.sample(lg, T, k, p, u)
        R = int(d.q.sum())
        # skip draws or cuts within rounding of a boundary (both sides round)
        if min(d.draw_margin, d.cut_margin) < 1e-9 * max(R, 1) + 64:
            continue
        assert d.token == _brute(lg, T, k, p, u), (lg, T, k, p, u)
        checked += 1
    assert checked > 2500
