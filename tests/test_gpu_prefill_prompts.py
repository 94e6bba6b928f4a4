"""GPU parity of qd_prefill_prompts (prompt chunks on the matrix cores)
against the CPU oracle, through the C ABI.

* Tiny shapes with every head layout the kernels take (head_dim 64 with 2 or
  1 query heads per KV head, head_dim 128 with 4): prompt segments packed
  into one chunk with ragged lengths (1 row; 300 rows = several GEMM row
  blocks and a ragged tail), continuation chunks whose earlier positions are
  already in the pool (start_pos > 0), and segments that end no prompt (no
  logits).  Each prompt's last logits and greedy id are checked against the
  oracle run one position at a time, to the decode step's bound.  Layer 0's
  appended K/V rows take the one-stage bound; deeper layers' rows are outputs
  of the whole stack below them and take the logits' end-to-end bound.  No
  other pool row may change.
* Qwen3-4B widths with 2 layers: one 512-row prompt.  This is the launch
  configuration the benchmark times: the GEMM tiles depend on the widths and
  the row count, not on the depth.  It is checked against
  ``Oracle.prefill_chunk``, whose projections are numpy matrix products.
* Prefill then decode: greedy decode steps continue from the prefilled pool,
  each checked against the oracle.
* Bad arguments come back as codes and launch nothing.  Out-of-pool
  block-table entries and out-of-vocabulary tokens are flagged, not
  faulting.
"""
import numpy as np
import pytest

import oracle
from paged_kv_gqa_qwen3_amd import binding, synth
from paged_kv_gqa_qwen3_amd.decoder import Decoder, pool_to_device, pool_to_host
from gpu_util import (LOGIT_RTOL, appended_mask, assert_kv_close, check_logits,
                      check_next_ids, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return _t


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


SHAPES = {
    "d64g2": synth.TINY,
    "d128g4": synth.ModelShape("d128g4", 2, 256, 8, 2, 128, 704, 4096, True),
    "d64g1": synth.ModelShape("d64g1", 2, 256, 2, 2, 64, 704, 4096, False),
}


def _run_calls(torch, dec, prompts, tables, pool, calls, V):
    """calls: [[(prompt, start, end), ...], ...]; in each call the segments
    that end their prompt come first and get logits.  Returns {prompt:
    (logits, next id)} from the GPU."""
    got = {}
    for ci, segs in enumerate(calls):
        n = 0
        while n < len(segs) and segs[n][2] == len(prompts[segs[n][0]]):
            n += 1
        assert not any(e == len(prompts[s]) for s, _, e in segs[n:])
        say(f"prefill_prompts call {ci}: segments {segs}, {n} with logits")
        tok = _i32(torch, np.concatenate([prompts[s][a:e] for s, a, e in segs]))
        tab = _i32(torch, tables[[s for s, _, _ in segs]])
        nxt = torch.full((max(n, 1),), -1, dtype=torch.int32, device="cuda")
        lg = torch.zeros(max(n, 1), V, dtype=torch.float32, device="cuda")
        dec.prefill_prompts([e - a for _, a, e in segs], [a for _, a, _ in segs], tok, tab, pool,
                            n, nxt if n else None, lg if n else None)
        torch.cuda.synchronize()
        for i in range(n):
            got[segs[i][0]] = (lg[i].cpu().numpy(), nxt[i:i + 1].cpu().numpy())
    return got


def _check_kv(host, pool_or, pool_start, mask, L):
    np.testing.assert_array_equal(host[~mask], pool_start[~mask])
    assert_kv_close(oracle.bf16_to_f64(host[0][mask[0]]), oracle.bf16_to_f64(pool_or[0][mask[0]]),
                    "prefill KV, layer 0")
    worst = 0.0
    for l in range(1, L):
        a, b = oracle.bf16_to_f64(host[l][mask[l]]), oracle.bf16_to_f64(pool_or[l][mask[l]])
        scale = np.abs(b).max(axis=-1, keepdims=True) + 1e-30
        r = np.abs(a - b) / (2.0 ** -7 * np.abs(b) + LOGIT_RTOL * scale)
        worst = max(worst, float(r.max()))
        assert np.all(r <= 1.0), f"prefill KV, layer {l}: worst ratio {float(r.max()):.3f}"
    say(f"prefill KV: worst end-to-end ratio {worst:.3f} (layers 1..{L - 1})")


PLANS = {
    # one long prompt: 300 rows, several 64/128-row GEMM blocks and a ragged tail
    "one_300": ([300], [[(0, 0, 300)]]),
    # four prompts in one chunk, all ending (a 1-row prompt among them)
    "four": ([70, 45, 1, 21], [[(0, 0, 70), (1, 0, 45), (2, 0, 1), (3, 0, 21)]]),
    # continuation chunks: earlier positions already in the pool; segments
    # that end no prompt get no logits
    "chunks": ([100, 40, 33], [[(1, 0, 40), (0, 0, 64), (2, 0, 10)],
                               [(2, 10, 33), (0, 64, 100)]]),
}


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("shape_name", list(SHAPES))
def test_tiny_prompts_match_oracle(torch, shape_name, plan):
    shape = SHAPES[shape_name]
    lens, calls = PLANS[plan]
    seed = 700 + sum(lens) + len(shape_name)
    W = synth.make_weights(shape, seed)
    prompts = [synth.uniform_int(seed + i, "prompt", shape.vocab, n) for i, n in enumerate(lens)]
    batch = synth.make_paged_batch(shape, [0] * len(lens), max(lens), seed, fill_kv=False)
    pool_start = batch.pool.copy()
    pool = pool_to_device(batch.pool)
    rows = max(sum(e - a for _, a, e in segs) for segs in calls)
    dec = Decoder(shape, 4, batch.max_pages, batch.num_pages, max_prefill_rows=rows)
    dec.load_numpy_weights(W)
    got = _run_calls(torch, dec, prompts, batch.block_tables, pool, calls, shape.vocab)
    assert dec.device_status() == 0
    dec.close()
    orc = oracle.Oracle(shape, W)
    pool_or = batch.pool
    for s, pr in enumerate(prompts):
        lg_or, _ = orc.prefill(pr, batch.block_tables[s], pool_or)
        r = check_logits(got[s][0][None], lg_or[None], f"prompt {s}")
        check_next_ids(got[s][1], lg_or[None], f"prompt {s}")
        say(f"{shape_name}/{plan} prompt {s} ({len(pr)} tokens): logit ratio {r:.3e}")
    m = appended_mask(batch, [(s, p) for s, pr in enumerate(prompts) for p in range(len(pr))])
    _check_kv(pool_to_host(pool), pool_or, pool_start, m, shape.num_layers)


def test_full_width_512_row_prompt(torch):
    """Qwen3-4B widths (2 layers): a 512-row prompt, last logits, greedy id and
    every appended K/V row against Oracle.prefill_chunk."""
    base = synth.QWEN3_4B
    shape = synth.ModelShape("qwen3-4b-2l", 2, base.hidden, base.num_q_heads,
                             base.num_kv_heads, base.head_dim, base.intermediate, base.vocab,
                             base.tie_embeddings)
    T = 512
    say("generating qwen3-4b-2l weights")
    W = synth.make_weights(shape, 9)
    prompt = synth.uniform_int(91, "prompt", shape.vocab, T)
    batch = synth.make_paged_batch(shape, [0], T, 9, fill_kv=False)
    pool_start = batch.pool.copy()
    pool = pool_to_device(batch.pool)
    dec = Decoder(shape, 1, batch.max_pages, batch.num_pages, max_prefill_rows=T)
    dec.load_numpy_weights(W)
    got = _run_calls(torch, dec, [prompt], batch.block_tables, pool, [[(0, 0, T)]], shape.vocab)
    assert dec.device_status() == 0
    dec.close()
    say("oracle: prefill_chunk of 512 rows")
    orc = oracle.Oracle(shape, W)
    order = np.r_[T - 1, np.arange(T - 1)]  # the head row (the prompt's last) first
    lg_or, _ = orc.prefill_chunk(prompt[order], order.astype(np.int32),
                                 np.repeat(batch.block_tables, T, axis=0), batch.pool, 1)
    r = check_logits(got[0][0][None], lg_or, "512-row prompt")
    check_next_ids(got[0][1], lg_or, "512-row prompt")
    say(f"512-row prompt: logit ratio {r:.3e}")
    m = appended_mask(batch, [(0, p) for p in range(T)])
    _check_kv(pool_to_host(pool), batch.pool, pool_start, m, shape.num_layers)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape_name", ["d64g2", "d128g4"])
def test_fp8_pool_prompts_match_oracle(torch, shape_name):
    """qd_prefill_prompts on an 8-bit (E4M3) pool, scales 0.5 for K and 2 for
    V: continuation chunks and segments that end no prompt, each prompt's last
    logits against the oracle on its own 8-bit pool, one position at a time;
    no other pool byte changes, and layer 0's codes are within one step of
    the oracle's (the two sides round values that differ by the projection's
    error only)."""
    shape = SHAPES[shape_name]
    kv = oracle.KvFormat(True, 0.5, 2.0)
    lens, calls = PLANS["chunks"]
    seed = 770 + len(shape_name)
    W = synth.make_weights(shape, seed)
    prompts = [synth.uniform_int(seed + i, "prompt", shape.vocab, n) for i, n in enumerate(lens)]
    batch = synth.make_paged_batch(shape, [0] * len(lens), max(lens), seed, fill_kv=False,
                                   kv_fp8=True)
    pool_start = batch.pool.copy()
    pool = pool_to_device(batch.pool)
    rows = max(sum(e - a for _, a, e in segs) for segs in calls)
    dec = Decoder(shape, 4, batch.max_pages, batch.num_pages, max_prefill_rows=rows,
                  kv_fp8=True, k_scale=kv.k_scale, v_scale=kv.v_scale)
    dec.load_numpy_weights(W)
    got = _run_calls(torch, dec, prompts, batch.block_tables, pool, calls, shape.vocab)
    assert dec.device_status() == 0
    dec.close()
    orc = oracle.Oracle(shape, W)
    pool_or = batch.pool
    for s, pr in enumerate(prompts):
        lg_or, _ = orc.prefill(pr, batch.block_tables[s], pool_or, kv=kv)
        r = check_logits(got[s][0][None], lg_or[None], f"prompt {s}")
        check_next_ids(got[s][1], lg_or[None], f"prompt {s}")
        say(f"fp8 {shape_name} prompt {s} ({len(pr)} tokens): logit ratio {r:.3e}")
    m = appended_mask(batch, [(s, p) for s, pr in enumerate(prompts) for p in range(len(pr))])
    host = pool_to_host(pool)
    np.testing.assert_array_equal(host[~m], pool_start[~m])
    # layer 0's codes come from the embedding through one projection: the
    # two sides' values differ by the projection's rounding only, so a code
    # may differ from the oracle's by one step where the value sits at a
    # rounding boundary, never more
    a, b = host[0][m[0]].astype(np.int32), pool_or[0][m[0]].astype(np.int32)
    same_sign = (a & 0x80) == (b & 0x80)
    assert np.all(same_sign | ((a & 0x7F) == 0) | ((b & 0x7F) == 0))
    assert np.abs((a & 0x7F) - (b & 0x7F)).max() <= 1
    say(f"fp8 {shape_name}: layer-0 codes equal {np.mean(a == b):.4f}")


def test_prompt_then_decode(torch):
    """A 40-token prompt through qd_prefill_prompts, then 8 greedy decode
    steps from its own next id, each checked against the oracle (which
    prefills one position at a time and decodes teacher-forced)."""
    shape = synth.TINY
    W = synth.make_weights(shape, 78)
    n, steps = 40, 8
    prompt = synth.uniform_int(78, "prompt", shape.vocab, n)
    batch = synth.make_paged_batch(shape, [0], n + steps, 78, fill_kv=False)
    table = batch.block_tables
    pool = pool_to_device(batch.pool)
    pool_or = batch.pool.copy()
    dec = Decoder(shape, 4, batch.max_pages, batch.num_pages, max_prefill_rows=64)
    dec.load_numpy_weights(W)
    got = _run_calls(torch, dec, [prompt], table, pool, [[(0, 0, n)]], shape.vocab)
    orc = oracle.Oracle(shape, W)
    lg_or, token = orc.prefill(prompt, table[0], pool_or)
    check_logits(got[0][0][None], lg_or[None], "prefill")
    check_next_ids(got[0][1], lg_or[None], "prefill")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    tab = _i32(torch, table)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
    for step in range(steps):
        say(f"prompt then decode: step {step}")
        tok.fill_(token)
        pos.fill_(n + step)
        dec.step(tok, pos, tab, pool, nxt, lg)
        lg_or, nx_or, _ = orc.decode_step(np.array([token], np.int32),
                                          np.array([n + step], np.int32), table, pool_or)
        torch.cuda.synchronize()
        check_logits(lg.cpu().numpy(), lg_or, f"step {step}")
        check_next_ids(nxt.cpu().numpy(), lg_or, f"step {step}")
        token = int(nx_or[0])
    assert dec.device_status() == 0
    dec.close()


def test_prompts_reject_bad_arguments(torch):
    """Argument errors come back as codes and launch nothing; device-side
    index errors are clamped and flagged."""
    shape = synth.TINY
    batch = synth.make_paged_batch(shape, [0, 0], 40, 5, fill_kv=False)
    pool = pool_to_device(batch.pool)
    tok = _i32(torch, np.arange(64) % shape.vocab)
    tab = _i32(torch, batch.block_tables)
    nxt = torch.zeros(4, dtype=torch.int32, device="cuda")
    W = synth.make_weights(shape, 5)

    plain = Decoder(shape, 4, batch.max_pages, batch.num_pages)
    plain.load_numpy_weights(W)
    with pytest.raises(binding.QdError) as e:
        plain.prefill_prompts([8], [0], tok, tab, pool, 1, nxt)
    assert e.value.code == binding.QD_EUNSUPPORTED
    plain.close()

    dec = Decoder(shape, 2, batch.max_pages, batch.num_pages, max_prefill_rows=48)
    with pytest.raises(binding.QdError) as e:  # weights not loaded
        dec.prefill_prompts([8], [0], tok, tab, pool, 1, nxt)
    assert e.value.code == binding.QD_ESTATE
    dec.load_numpy_weights(W)
    bad = [
        ([], [], 0),                 # no segment
        ([0], [0], 0),               # empty segment
        ([8], [-1], 0),              # negative start
        ([8], [batch.max_pages * 16 - 4], 0),  # runs past the block table
        ([30, 19], [0, 0], 0),       # 49 rows > max_prefill_rows
        ([8], [0], 2),               # n_logits > n_seqs
        ([8, 8, 8], [0, 0, 0], 3),   # n_logits > max_batch
    ]
    for rows, starts, n in bad:
        with pytest.raises(binding.QdError) as e:
            dec.prefill_prompts(rows, starts, tok, tab, pool, n, nxt)
        assert e.value.code == binding.QD_EINVAL, (rows, starts, n)
    with pytest.raises(binding.QdError):  # logits asked, no next-id output
        dec.prefill_prompts([8], [0], tok, tab, pool, 1, None)
    with pytest.raises(binding.QdError):
        binding.qd_prefill_prompts(dec.handle, [1] * 65, [0] * 65, tok, tab, pool, 0)
    torch.cuda.synchronize()
    assert dec.device_status() == 0
    # a block-table entry outside the pool and a token outside the vocabulary
    bt = batch.block_tables.copy()
    bt[0, 1] = batch.num_pages + 3
    bad_tok = tok.clone()
    bad_tok[3] = shape.vocab + 7
    dec.prefill_prompts([20], [0], bad_tok, _i32(torch, bt), pool, 1, nxt)
    torch.cuda.synchronize()
    st = dec.device_status()
    assert st & binding.QD_DEV_BAD_PAGE and st & binding.QD_DEV_BAD_TOKEN, st
    dec.close()
