"""GPU tests of the continuous-batching serving loop (qd_engine_* through the
C ABI) against the CPU oracle.

Requests arrive at different iterations, with ragged prompts (1 to 130
tokens; with 64 prompt rows per iteration the long ones are prefilled over
several iterations), shared prefixes, an end-of-sequence id and more
requests than the batch holds, so the decode batch size changes from one
iteration to the next and each size replays its own graph.  Every token a
request returns is checked against the oracle run teacher-forced on that
request's own tokens (its prompt one position at a time, then one decode
step per returned token), to the decode step's greedy rule; the request
ends exactly at its limit or its end-of-sequence token; no request returns
two tokens in one iteration; and when everything is done every page of the
pool is obtainable again.  The prefix cache must have supplied prompt pages
(a request whose prompt repeats a finished one's).  Variants: graphs for
every batch size, the weight-streaming kernel at batch 1, an 8-bit E4M3
pool, a pool so small that requests wait for pages, and a batch limit of 24
(decode batches past 16 columns).
"""
import numpy as np
import pytest

import oracle
from paged_kv_gqa_qwen3_amd import binding, synth
from paged_kv_gqa_qwen3_amd.decoder import Decoder, pool_to_device
from gpu_util import check_next_ids, say

pytestmark = pytest.mark.gpu

SHAPE = synth.TINY
PAGE = 16


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return _t


def _requests(seed):
    """{iteration: [(request id, prompt, max_new_tokens, eos)]} and the prompts."""
    V = SHAPE.vocab
    sys_prefix = synth.uniform_int(seed, "system", V, 40)
    tail = lambda name, n: synth.uniform_int(seed, name, V, n)
    a = np.concatenate([sys_prefix, tail("a", 30)])
    plan = {
        0: [(10, a, 9, -1), (11, tail("b", 5), 14, -1), (12, tail("c", 130), 6, -1),
            (13, tail("d", 1), 4, -1)],
        2: [(14, np.concatenate([sys_prefix, tail("e", 7)]), 6, -1)],
        # eos: filled in from the oracle; this prompt's greedy run changes
        # token at a decode step (most prompts of this random model repeat
        # their first token)
        5: [(16, tail("g24", 20), 8, None)],
        15: [(17, np.concatenate([sys_prefix, tail("h", 3)]), 7, -1)],
        # once request 10 has left: its prompt again, whose first 64
        # positions are then in the prefix cache
        ("after", 10): [(15, a.copy(), 5, -1)],
    }
    return plan


def _oracle_greedy(orc, prompt, n, kv):
    """The oracle's own greedy continuation of a prompt (n tokens)."""
    batch = synth.make_paged_batch(SHAPE, [0], len(prompt) + n, 5, fill_kv=False,
                                   kv_fp8=kv.fp8)
    pool = batch.pool
    row = batch.block_tables[:1]
    _, tok = orc.prefill(prompt, row[0], pool, kv=kv)
    out = [tok]
    for k in range(1, n):
        _, nx, _ = orc.decode_step(np.array([tok], np.int32), np.array([len(prompt) + k - 1], np.int32),
                                   row, pool, kv=kv)
        tok = int(nx[0])
        out.append(tok)
    return out


def _drive(torch, eng, plan, max_iters=200):
    """Run iterations until every request is done.  Returns the streams, the
    iteration each request ended in, the decode batch size of every
    iteration and the final stats."""
    streams, finished, per_iter = {}, {}, []
    last = max(k for k in plan if isinstance(k, int))
    follow = {k[1]: v for k, v in plan.items() if not isinstance(k, int)}
    it = 0
    decoded = 0
    while True:
        todo = list(plan.get(it, []))
        for r in [r for r in follow if r in finished]:
            todo += follow.pop(r)
        for req, prompt, mx, eos in todo:
            eng.submit(req, prompt, mx, eos)
        out = eng.step()
        seen = set()
        for r, t, d in out:
            assert r not in seen, f"iteration {it}: request {r} returned two tokens"
            assert r not in finished, f"iteration {it}: request {r} returned a token after its end"
            seen.add(r)
            streams.setdefault(r, []).append(t)
            if d:
                finished[r] = it
        st = eng.stats()
        per_iter.append(st["decode_rows"] - decoded)
        decoded = st["decode_rows"]
        it += 1
        if it > last and not follow and st["waiting"] == 0 and st["running"] == 0:
            return streams, finished, per_iter, st
        assert it < max_iters, "the engine did not finish its requests"


def _check_streams(orc, plan, streams, finished, kv):
    reqs = [x for v in plan.values() for x in v]
    ctx = max(len(p) + mx for _, p, mx, _ in reqs)
    batch = synth.make_paged_batch(SHAPE, [0] * len(reqs), ctx, 9, fill_kv=False, kv_fp8=kv.fp8)
    pool = batch.pool
    excused = 0
    for i, (req, prompt, mx, eos) in enumerate(reqs):
        got = streams[req]
        assert req in finished, f"request {req} never finished"
        assert 1 <= len(got) <= mx
        assert all(t != eos for t in got[:-1]), f"request {req} went past its eos"
        assert len(got) == mx or got[-1] == eos, f"request {req} stopped early"
        row = batch.block_tables[i:i + 1]
        lg, _ = orc.prefill(prompt, row[0], pool, kv=kv)
        excused += check_next_ids(np.array(got[:1]), lg[None], f"request {req} token 0")
        for k in range(1, len(got)):
            lg, _, _ = orc.decode_step(np.array([got[k - 1]], np.int32),
                                       np.array([len(prompt) + k - 1], np.int32), row, pool, kv=kv)
            excused += check_next_ids(np.array([got[k]]), lg, f"request {req} token {k}")
        say(f"request {req}: prompt {len(prompt)}, {len(got)} tokens, ended at iteration "
            f"{finished[req]}")
    return excused


VARIANTS = {
    "graphs": dict(persistent=False, kv_fp8=False),
    "stream_b1": dict(persistent=True, kv_fp8=False),
    "fp8_pool": dict(persistent=False, kv_fp8=True),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_engine_matches_oracle(torch, variant):
    opts = VARIANTS[variant]
    kv = oracle.KvFormat(True, 0.5, 0.25) if opts["kv_fp8"] else oracle.BF16
    seed = 901
    W = synth.make_weights(SHAPE, seed)
    orc = oracle.Oracle(SHAPE, W)
    plan = _requests(seed)
    # request 16 ends on a token that the oracle's own greedy run reaches
    # first at a decode step (its second token or later)
    g_prompt = plan[5][0][1]
    greedy = _oracle_greedy(orc, g_prompt, 7, kv)
    eos = next(t for k, t in enumerate(greedy) if k >= 1 and t not in greedy[:k])
    plan[5] = [(16, g_prompt, 8, eos)]
    say(f"{variant}: request 16 eos id {eos}")

    num_pages, mpps = 64, 16
    dtype = np.uint8 if opts["kv_fp8"] else np.uint16
    pool = pool_to_device(np.zeros((SHAPE.num_layers, num_pages, 2, SHAPE.num_kv_heads, PAGE,
                                    SHAPE.head_dim), dtype=dtype))
    dec = Decoder(SHAPE, 4, mpps, num_pages, persistent=opts["persistent"], max_prefill_rows=64,
                  kv_fp8=opts["kv_fp8"], k_scale=kv.k_scale, v_scale=kv.v_scale)
    dec.load_numpy_weights(W)
    if opts["persistent"]:
        assert dec.step_path(1) == "stream"
    eng = binding.Engine(dec.handle, pool, 4)
    streams, finished, per_iter, st = _drive(torch, eng, plan)
    say(f"{variant}: decode batch per iteration {per_iter}")
    say(f"{variant}: stats {st}")
    assert st["pages_available"] == num_pages
    # request 15 takes 4 pages of request 10's prompt, request 17 the two
    # full pages of the shared 40-token prefix
    assert st["cached_rows"] == 64 + 32, "the prefix cache did not supply the expected pages"
    assert st["tokens_out"] == sum(len(s) for s in streams.values())
    assert len(set(per_iter) - {0}) >= 4, "the decode batch did not take sizes 1 to 4"
    eng.close()
    assert dec.device_status() == 0
    dec.close()
    excused = _check_streams(orc, plan, streams, finished, kv)
    say(f"{variant}: {excused} near-tie ids excused")
    assert streams[16][-1] == eos and len(streams[16]) < 8, "request 16 did not end on its eos"


def test_engine_wide_batches(torch):
    """30 requests through a batch limit of 24: the decode batch grows past
    16 columns (the chunk-streamed 32-column GEMV items and their shared
    split reductions) and shrinks again as requests end, each size on its
    own graph; every stream is still the oracle's."""
    seed = 903
    W = synth.make_weights(SHAPE, seed)
    orc = oracle.Oracle(SHAPE, W)
    V = SHAPE.vocab
    plan = {}
    rid = 100
    for it, n in ((0, 10), (1, 8), (2, 8), (4, 4)):
        reqs = []
        for _ in range(n):
            plen = 3 + (rid * 7) % 37
            reqs.append((rid, synth.uniform_int(seed, f"w{rid}", V, plen), 5 + rid % 6, -1))
            rid += 1
        plan[it] = reqs
    num_pages, mpps = 96, 4
    pool = pool_to_device(np.zeros((SHAPE.num_layers, num_pages, 2, SHAPE.num_kv_heads, PAGE,
                                    SHAPE.head_dim), dtype=np.uint16))
    dec = Decoder(SHAPE, 24, mpps, num_pages, max_prefill_rows=256)
    dec.load_numpy_weights(W)
    eng = binding.Engine(dec.handle, pool, 24)
    streams, finished, per_iter, st = _drive(torch, eng, plan)
    say(f"wide: decode batch per iteration {per_iter}")
    assert max(per_iter) > 16, "the decode batch never passed 16"
    assert st["pages_available"] == num_pages
    assert st["tokens_out"] == sum(len(s) for s in streams.values())
    eng.close()
    assert dec.device_status() == 0
    dec.close()
    excused = _check_streams(orc, plan, streams, finished, oracle.BF16)
    say(f"wide: {excused} near-tie ids excused")


def test_engine_waits_for_pages(torch):
    """A 14-page pool: requests take all their pages when admitted, so only
    some fit at once; the others wait in line and every stream is still the
    oracle's."""
    seed = 902
    W = synth.make_weights(SHAPE, seed)
    orc = oracle.Oracle(SHAPE, W)
    V = SHAPE.vocab
    plan = {0: [(1, synth.uniform_int(seed, "p1", V, 90), 10, -1),     # 7 pages
                (2, synth.uniform_int(seed, "p2", V, 60), 12, -1),     # 5 pages
                (3, synth.uniform_int(seed, "p3", V, 30), 20, -1),     # 4 pages
                (4, synth.uniform_int(seed, "p4", V, 150), 4, -1)],    # 10 pages
            1: [(5, synth.uniform_int(seed, "p5", V, 17), 3, -1)]}     # 2 pages
    num_pages, mpps = 14, 12
    pool = pool_to_device(np.zeros((SHAPE.num_layers, num_pages, 2, SHAPE.num_kv_heads, PAGE,
                                    SHAPE.head_dim), dtype=np.uint16))
    dec = Decoder(SHAPE, 4, mpps, num_pages, max_prefill_rows=96)
    dec.load_numpy_weights(W)
    eng = binding.Engine(dec.handle, pool, 4)
    streams, finished, per_iter, st = _drive(torch, eng, plan)
    say(f"waits_for_pages: decode batch per iteration {per_iter}, stats {st}")
    assert st["pages_available"] == num_pages
    assert max(per_iter) < 4, "requests that cannot all fit ran together"
    eng.close()
    assert dec.device_status() == 0
    dec.close()
    _check_streams(orc, plan, streams, finished, oracle.BF16)


def test_engine_rejects_bad_requests(torch):
    num_pages, mpps = 8, 4
    pool = pool_to_device(np.zeros((SHAPE.num_layers, num_pages, 2, SHAPE.num_kv_heads, PAGE,
                                    SHAPE.head_dim), dtype=np.uint16))
    W = synth.make_weights(SHAPE, 3)
    plain = Decoder(SHAPE, 2, mpps, num_pages)
    with pytest.raises(binding.QdError) as e:
        binding.Engine(plain.handle, pool, 2)
    assert e.value.code == binding.QD_EUNSUPPORTED
    plain.close()
    dec = Decoder(SHAPE, 2, mpps, num_pages, max_prefill_rows=32)
    dec.load_numpy_weights(W)
    eng = binding.Engine(dec.handle, pool, 2)
    ok = np.arange(5, dtype=np.int32)
    cases = [((1, [], 4, -1), binding.QD_EINVAL),                      # empty prompt
             ((1, ok, 0, -1), binding.QD_EINVAL),                      # no tokens wanted
             ((1, [0, SHAPE.vocab], 4, -1), binding.QD_EINVAL),        # token outside the vocabulary
             ((1, ok, 4, SHAPE.vocab), binding.QD_EINVAL),             # eos outside the vocabulary
             ((1, np.zeros(60, np.int32), 10, -1), binding.QD_EUNSUPPORTED)]  # past 4 pages
    for args, code in cases:
        with pytest.raises(binding.QdError) as e:
            eng.submit(*args)
        assert e.value.code == code, args
    eng.submit(1, ok, 3)
    with pytest.raises(binding.QdError) as e:
        eng.submit(1, ok, 3)  # id in use
    assert e.value.code == binding.QD_EINVAL
    out = []
    while True:
        got = eng.step()
        out += got
        if not got:
            break
    assert [r for r, _, _ in out] == [1, 1, 1] and out[-1][2]
    st = eng.stats()
    assert st["running"] == 0 and st["pages_available"] == num_pages
    eng.close()
    assert dec.device_status() == 0
    dec.close()


def _plain_plan(seed, n=6):
    """n requests at iteration 0 and 2, prompts of 9..60 tokens, 10 new tokens."""
    V = SHAPE.vocab
    reqs = [(100 + i, synth.uniform_int(seed, f"s{i}", V, 9 + 11 * i), 10) for i in range(n)]
    return reqs


def _run_engine(torch, W, reqs, opts, num_pages=64, mpps=8):
    pool = pool_to_device(np.zeros((SHAPE.num_layers, num_pages, 2, SHAPE.num_kv_heads, PAGE,
                                    SHAPE.head_dim), dtype=np.uint16))
    dec = Decoder(SHAPE, 4, mpps, num_pages, max_prefill_rows=64)
    dec.load_numpy_weights(W)
    eng = binding.Engine(dec.handle, pool, 4)
    for i, (rid, prompt, mx) in enumerate(reqs):
        eng.submit(rid, prompt, mx, **opts(i))
    streams = {}
    while True:
        out = eng.step()
        for r, t, d in out:
            streams.setdefault(r, []).append(t)
        st = eng.stats()
        if st["waiting"] == 0 and st["running"] == 0:
            break
    eng.close()
    assert dec.device_status() == 0
    dec.close()
    return streams, st


def test_engine_top1_sampling_equals_greedy(torch):
    """Requests that sample with top_k = 1 (any temperature) get the greedy
    streams exactly: the iterations then run qd_sample on the steps' logits
    instead of taking the steps' argmax, and both pick the lowest index of
    the largest logit."""
    W = synth.make_weights(SHAPE, 903)
    reqs = _plain_plan(903)
    greedy, st_g = _run_engine(torch, W, reqs, lambda i: {})
    top1, st_s = _run_engine(torch, W, reqs,
                             lambda i: dict(temperature=0.7 + 0.1 * i, top_k=1, seed=i))
    assert st_g["sampled_iterations"] == 0 and st_s["sampled_iterations"] == st_s["steps"]
    assert top1 == greedy


def test_engine_sampling_valid_and_reproducible(torch):
    """Greedy and sampling requests in one batch (temperature 1, top_k 5;
    one with top_p 0.9): greedy streams follow the oracle's argmax, every
    sampled token is among the oracle's 5 largest logits (teacher-forced on
    the request's own tokens, within the logit tolerance), sampling does not
    always pick the argmax, and a second run with the same seeds returns the
    same streams."""
    W = synth.make_weights(SHAPE, 904)
    orc = oracle.Oracle(SHAPE, W)
    reqs = _plain_plan(904)

    def opts(i):
        if i % 3 == 0:
            return {}
        if i == 5:
            return dict(temperature=1.0, top_p=0.9, seed=1000 + i)
        return dict(temperature=1.0, top_k=5, seed=1000 + i)
    s1, st = _run_engine(torch, W, reqs, opts)
    s2, _ = _run_engine(torch, W, reqs, opts)
    assert s1 == s2, "the same seeds gave different streams"
    assert st["sampled_iterations"] > 0
    batch = synth.make_paged_batch(SHAPE, [0] * len(reqs), 80, 11, fill_kv=False)
    pool = batch.pool
    off_argmax = 0
    for i, (rid, prompt, mx) in enumerate(reqs):
        got = s1[rid]
        assert len(got) == mx
        row = batch.block_tables[i:i + 1]
        lg, _ = orc.prefill(prompt, row[0], pool)
        lgs = [lg]
        for k in range(1, len(got)):
            l2, _, _ = orc.decode_step(np.array([got[k - 1]], np.int32),
                                       np.array([len(prompt) + k - 1], np.int32), row, pool)
            lgs.append(l2[0])
        for k, (t, l) in enumerate(zip(got, lgs)):
            if i % 3 == 0:
                check_next_ids(np.array([t]), l[None], f"greedy request {rid} token {k}")
                continue
            tol = 2e-2 * np.abs(l).max()
            off_argmax += int(t != int(np.argmax(l)))
            if i != 5:
                fifth = np.sort(l)[-5]
                assert l[t] >= fifth - tol, f"request {rid} token {k}: {t} outside the top 5"
        say(f"request {rid}: {got}")
    say(f"sampled tokens off the argmax: {off_argmax}")
    assert off_argmax > 0, "sampling never left the argmax"
