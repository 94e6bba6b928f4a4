"""GPU parity of on-device sampling (qd_sample) against the sampling oracle.

The kernel computes each weight in fp32 (exp of (logit - max) / T) and the
oracle in fp64, so their integer weights may differ by about 2^-18 of a
weight plus one unit.  A draw is compared exactly wherever the oracle's
draw target and top-p cut lie farther than that bound (summed over the
kept tokens, with a factor of 2) from a boundary; otherwise the GPU's token
must still be one the filters keep (or the token just past the top-p cut).
The top-k filter involves no arithmetic: a kept token is checked exactly.
"""
import numpy as np
import pytest

from oracle import sampling as S
from paged_kv_gqa_qwen3_amd import binding, synth
from paged_kv_gqa_qwen3_amd.decoder import Decoder, pool_to_device
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return _t


def _handle(vocab, max_batch=64):
    shape = synth.ModelShape(f"v{vocab}", 2, 256, 4, 2, 64, 704, vocab, True)
    return Decoder(shape, max_batch, 4, 8)


def _run(torch, dec, logits, T, k, p, u):
    dev = "cuda"
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    B = lg.shape[0]
    out = torch.full((B,), -7, dtype=torch.int32, device=dev)
    dec.sample(lg, torch.tensor(T, dtype=torch.float32, device=dev),
               torch.tensor(k, dtype=torch.int32, device=dev),
               torch.tensor(p, dtype=torch.float32, device=dev),
               torch.tensor(u, dtype=torch.float32, device=dev), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(logits, T, k, p, u, got):
    """Exact where the oracle's draw is clear of rounding, valid otherwise;
    returns the number of draws compared exactly."""
    exact = 0
    for r in range(len(got)):
        d = S.sample(logits[r], T[r], k[r], p[r], u[r])
        R = int(d.q.sum())
        tol = 2 * (R * 2.0 ** -18 + int(d.kept.sum()) + 1)
        g = int(got[r])
        assert 0 <= g < logits.shape[1], (r, g)
        if T[r] > 0 and 0 < k[r] < logits.shape[1]:
            order = S.rank_order(logits[r])
            assert g in set(order[:k[r]].tolist()), (r, "outside top-k")
        if d.draw_margin > tol and d.cut_margin > tol:
            assert g == d.token, (r, T[r], k[r], p[r], u[r], g, d.token)
            exact += 1
        else:
            ok = set(np.flatnonzero(d.kept).tolist())
            if d.cut_margin <= tol:  # the cut may fall one token later
                order = S.rank_order(logits[r])
                n = int(d.kept.sum())
                ok |= set(order[:n + 1].tolist())
            assert g in ok, (r, g, d.token)
    return exact


def _rows(rng, V, n):
    """Logit rows: peaked normals, coarse values with many ties, flat rows,
    and the near-uniform spread of a randomly initialised model."""
    rows = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            rows.append(rng.normal(scale=rng.choice([2.0, 6.0]), size=V))
        elif kind == 1:
            rows.append(np.round(rng.normal(scale=3.0, size=V) * 2) / 2)
        elif kind == 2:
            rows.append(np.full(V, rng.normal()))
        else:
            rows.append(rng.normal(scale=0.05, size=V))
    return np.array(rows, np.float32)


@pytest.mark.parametrize("V", [4096, 151936])
def test_sample_matches_oracle(torch, V):
    rng = np.random.default_rng(V)
    dec = _handle(V)
    total = exact = 0
    for rep in range(3):
        B = 64 if V == 4096 else 24
        logits = _rows(rng, V, B)
        T = rng.choice([0.0, 0.5, 1.0, 1.7], size=B).astype(np.float32)
        k = rng.choice([0, 1, 2, 5, 50, 64, 65, 1000, V, -3], size=B).astype(np.int32)
        p = rng.choice([1.0, 0.95, 0.5, 0.1, 0.0], size=B).astype(np.float32)
        u = rng.random(B).astype(np.float32)
        say(f"sample V={V} rep {rep}")
        got = _run(torch, dec, logits, T, k, p, u)
        exact += _check(logits, T.astype(float), k, p.astype(float), u.astype(float), got)
        total += B
    say(f"V={V}: {exact} of {total} draws compared exactly")
    assert exact >= 0.8 * total
    dec.close()


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.7, 40, 1.0), (1.2, 0, 0.9), (0.9, 300, 0.6), (0.6, 20, 0.95)])
def test_sample_grid_of_draws(torch, T, k, p):
    """64 draws on a grid of u per launch, eight launches: the counts of each
    token follow the oracle's integer weights."""
    V = 4096
    rng = np.random.default_rng(17)
    row = rng.normal(scale=1.5, size=V).astype(np.float32)
    dec = _handle(V)
    logits = np.repeat(row[None], 64, axis=0)
    counts = np.zeros(V, int)
    n = 0
    for g in range(8):
        u = ((np.arange(64) * 8 + g + 0.5) / 512).astype(np.float32)
        got = _run(torch, dec, logits, [T] * 64, [k] * 64, [p] * 64, u)
        _check(logits, [T] * 64, [k] * 64, [p] * 64, u.astype(float), got)
        np.add.at(counts, got, 1)
        n += 64
    d = S.sample(row, T, k, p, 0.5)
    expect = n * d.q / d.q.sum()
    say(f"grid T={T} k={k} p={p}: {int(d.kept.sum())} tokens kept, "
        f"max count error {np.abs(counts - expect).max():.2f}")
    assert np.all(np.abs(counts - expect) <= 2.0)
    dec.close()


def test_sample_third_launch_rows_together(torch):
    """Whole batches of the rows the multi-workgroup radix selection takes at
    V = 151,936: top-p without a top-k limit, most with nuclei beyond the
    row's first 64 tokens, and top_k above 64 with and without top-p.  Every
    row against the oracle, on consecutive calls of different batch sizes
    that share the handle's histograms and counters, and a repeat of the
    first call giving the same ids."""
    V = 151936
    rng = np.random.default_rng(5150)
    dec = _handle(V)
    runs = []
    total = exact = beyond = 0
    for B in (64, 37):
        logits = _rows(rng, V, B)
        T = rng.choice([0.6, 1.0, 1.7], size=B).astype(np.float32)
        k = rng.choice([0, V, -5, 100, 3000], size=B).astype(np.int32)
        p = rng.choice([0.2, 0.5, 0.9, 0.99, 1.0], size=B).astype(np.float32)
        p[(k <= 0) | (k >= V)] = np.minimum(p[(k <= 0) | (k >= V)], 0.99)  # top-p or top-k
        u = rng.random(B).astype(np.float32)
        say(f"third-launch rows, batch {B}")
        got = _run(torch, dec, logits, T, k, p, u)
        exact += _check(logits, T.astype(float), k, p.astype(float), u.astype(float), got)
        beyond += sum(int(S.sample(logits[r], float(T[r]), int(k[r]), float(p[r]),
                                   float(u[r])).kept.sum()) > 64 for r in range(B))
        total += B
        runs.append((logits, T, k, p, u, got))
    logits, T, k, p, u, first = runs[0]
    again = _run(torch, dec, logits, T, k, p, u)
    np.testing.assert_array_equal(again, first)
    say(f"third launch: {beyond} of {total} rows keep more than 64 tokens, "
        f"{exact} compared exactly")
    assert beyond >= total // 2
    # flat and near-uniform rows put most of their cuts within the fp32
    # bound of a boundary (49 of these 101 draws are clear of it)
    assert exact >= total // 3
    dec.close()


def _edge_rows(rng, V):
    """Settings at the edges of the multi-workgroup selection: top-k just
    above the 64-token lists and at V - 1, a top-p cut at the first token,
    masked vocabularies (-inf logits: weight 0, still counted by top-k), a
    temperature that leaves nearly all weight on the maximum, near-uniform
    rows and coarse ties."""
    base = lambda: rng.normal(scale=2.0, size=V)
    masked = lambda: np.where(rng.random(V) < 0.5, -np.inf, rng.normal(scale=2.0, size=V))
    spike = lambda: np.where(np.arange(V) == V // 3, 8.0, rng.normal(scale=0.5, size=V))
    rows = [  # logits, T, top_k, top_p
        (base(), 1.0, 65, 1.0),
        (base(), 1.0, V - 1, 1.0),
        (base(), 0.8, V - 1, 0.999),
        (base(), 1.0, 1000, 1e-6),
        (masked(), 1.0, (3 * V) // 4, 1.0),
        (masked(), 1.2, 0, 0.9),
        (base(), 1e-3, 1000, 0.9),
        (rng.normal(scale=0.05, size=V), 2.0, 300, 0.5),
        (spike(), 1.0, 0, 0.99),
        (np.round(base() * 2) / 2, 1.0, 5000, 1.0),
    ]
    logits = np.array([r[0] for r in rows], np.float32)
    T = np.array([r[1] for r in rows], np.float32)
    k = np.array([r[2] for r in rows], np.int32)
    p = np.array([r[3] for r in rows], np.float32)
    return logits, T, k, p


@pytest.mark.parametrize("V", [4160, 32896, 151936])
def test_sample_third_launch_edge_cases(torch, V):
    """The edge settings against the oracle at one, five and nineteen chunks
    per row, twice with the rows in a different order (the second call
    finds the first call's histograms and counters cleared)."""
    rng = np.random.default_rng(V + 1)
    dec = _handle(V)
    logits, T, k, p = _edge_rows(rng, V)
    u = rng.random(len(T)).astype(np.float32)
    for call, perm in enumerate([np.arange(len(T)), rng.permutation(len(T))]):
        say(f"edge settings V={V} call {call}")
        got = _run(torch, dec, logits[perm], T[perm], k[perm], p[perm], u[perm])
        _check(logits[perm], T[perm].astype(float), k[perm], p[perm].astype(float),
               u[perm].astype(float), got)
        d = S.sample(logits[3], float(T[3]), int(k[3]), float(p[3]), float(u[3]))
        assert got[list(perm).index(3)] == d.token == S.rank_order(logits[3])[0]
    dec.close()


def test_sample_greedy_equals_step_argmax(torch):
    """Temperature 0, top_k 1 and top_p 0 all give the step's own argmax."""
    shape = synth.TINY
    W = synth.make_weights(shape, 61)
    batch = synth.make_paged_batch(shape, [3, 40, 90, 200, 7], 1, 62)
    B = 5
    dec = Decoder(shape, B, batch.max_pages, batch.num_pages)
    dec.load_numpy_weights(W)
    dev = "cuda"
    logits = torch.zeros(B, shape.vocab, device=dev)
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)
    pool = pool_to_device(batch.pool)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    dec.step(i32(batch.tokens), i32(batch.positions), i32(batch.block_tables), pool, nxt, logits)
    torch.cuda.synchronize()
    want = nxt.cpu().numpy()
    lg = logits.cpu().numpy()
    for T, k, p in ((0.0, 0, 1.0), (1.0, 1, 1.0), (0.8, 0, 0.0)):
        got = _run(torch, dec, lg, [T] * B, [k] * B, [p] * B, [0.9] * B)
        np.testing.assert_array_equal(got, want)
    dec.close()


def test_sample_rejects_bad_arguments(torch):
    dec = _handle(4096, max_batch=4)
    x = torch.zeros(4, 4096, device="cuda")
    f = torch.zeros(4, device="cuda")
    i = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.QdError):
        binding.qd_sample(dec.handle, 5, x, f, i, f, f, i)
    with pytest.raises(binding.QdError):
        binding.qd_sample(dec.handle, 0, x, f, i, f, f, i)
    with pytest.raises(binding.QdError):
        binding.qd_sample(dec.handle, 2, x, f, i, None, f, i)
    dec.close()
