"""CPU oracle for on-device sampling of the next token (temperature, top-k,
top-p).  The yuzheng310 page ("GPU 算子与执行优化", part 3, the host-overhead
battle) requires argmax and the top-p/top-k filters to run on the GPU so that
only the token id is written out; the rkmt page ("从零构建 Qwen3-8B 推理引擎",
section 4.1.2, the gRPC interface) passes temperature and top_p with a
request and returns the sampled token.

TEST INFRASTRUCTURE ONLY: the tests may use it; the GPU library never does.
It shares no code with the GPU path.  Plain numpy, fp64 for the weights.

The pages name the filters but fix no algorithm, so this follows the plain
definitions (the readings are listed with the library's design notes):

1. temperature <= 0: greedy, the lowest index among the largest logits.
2. Weights w_i = exp((l_i - max l) / T): softmax numerators; the
   normalisation does not change the distribution.
3. Rank order: logit descending, token id ascending.
4. top_k > 0: keep the first top_k tokens in rank order (0 or >= vocab: all).
5. top_p < 1: of the kept tokens, keep the shortest rank-order prefix whose
   weight sum reaches top_p times the kept weight sum.
6. Weights are summed as integers q_i = floor(w_i * 2^32), so that every sum
   is exact and independent of order; the top-p target is ceil(top_p * Q)
   and the draw target t = min(floor(u * R), R - 1), both formed in fp64.
7. The caller supplies u in [0, 1) per sequence; the sampled token is the
   kept token, in increasing id order, at which the running sum of q first
   exceeds t.
"""
from __future__ import annotations

import math
from typing import NamedTuple

import numpy as np

SCALE = 2.0 ** 32


class Draw(NamedTuple):
    token: int
    kept: np.ndarray      # bool [V]: the tokens left after top-k and top-p
    q: np.ndarray         # int64 [V]: integer weights (0 where not kept)
    target: int           # t, the draw target
    cut_margin: int       # top-p: |prefix sum at the cut - target| (large when unused)
    draw_margin: int      # min distance of t to the chosen token's interval ends


def rank_order(logits) -> np.ndarray:
    """Token ids by logit descending, then id ascending (reading 3)."""
    lg = np.asarray(logits, dtype=np.float64)
    return np.lexsort((np.arange(lg.size), -lg))


def weights_q(logits, temperature: float) -> np.ndarray:
    """Integer weights floor(exp((l - max) / T) * 2^32) (readings 2 and 6)."""
    lg = np.asarray(logits, dtype=np.float64)
    w = np.exp((lg - lg.max()) / float(temperature))
    return np.floor(w * SCALE).astype(np.int64)


def sample(logits, temperature: float, top_k: int, top_p: float, u: float) -> Draw:
    """One draw from the filtered, renormalised distribution of `logits`."""
    lg = np.asarray(logits, dtype=np.float64)
    V = lg.size
    big = 1 << 62
    if not temperature > 0.0:
        tok = int(np.argmax(lg))  # numpy returns the first index of the maximum
        kept = np.zeros(V, bool)
        kept[tok] = True
        return Draw(tok, kept, kept.astype(np.int64), 0, big, big)
    order = rank_order(lg)
    kept = np.ones(V, bool)
    if 0 < top_k < V:
        kept[:] = False
        kept[order[:top_k]] = True
    q = weights_q(lg, temperature)
    q = np.where(kept, q, 0)
    cut_margin = big
    if top_p < 1.0:
        Q = int(q.sum())
        target = int(math.ceil(float(top_p) * float(Q)))
        prefix = np.cumsum(q[order])  # rank order; dropped tokens add 0
        n = int(np.searchsorted(prefix, target, side="left")) + 1  # shortest prefix >= target
        n = max(1, min(n, V))
        keep2 = np.zeros(V, bool)
        keep2[order[:n]] = True
        kept &= keep2
        q = np.where(kept, q, 0)
        cut_margin = abs(int(prefix[n - 1]) - target)
        if n >= 2:
            cut_margin = min(cut_margin, abs(int(prefix[n - 2]) - target))
    R = int(q.sum())
    t = min(int(math.floor(float(u) * float(R))), R - 1)
    csum = np.cumsum(q)  # increasing token id
    tok = int(np.searchsorted(csum, t, side="right"))
    lo = int(csum[tok] - q[tok])
    draw_margin = min(t - lo, int(csum[tok]) - 1 - t)
    return Draw(tok, kept, q, t, cut_margin, draw_margin)
