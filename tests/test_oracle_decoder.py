"""Pins for the oracle's whole decode step (tiny shapes, CPU only).

* A full-sequence causal forward built from library routines (torch
  ``rms_norm``, ``linear``, ``scaled_dot_product_attention(is_causal=True,
  enable_gqa=True)``, ``silu``) must give the logits the oracle produces when
  it decodes the same prompt one position at a time through the paged pool.
  This pins the layer wiring (pre-norm residuals, q/k norm before RoPE, KV
  append before attention, causal inclusive context, tied LM head, final norm).
  ``Oracle.prefill`` is pinned by the same forward: its logits and greedy id
  are those of the prompt's last position, and the pool it fills holds the
  same bytes as the step-by-step loop's.  ``Oracle.prefill_chunk`` (a chunk's
  rows as one batch, projections as numpy matrix products) gives every row's
  logits of that forward, and agrees with ``decode_step`` on a continuation
  chunk of shuffled rows from two sequences.
* With the attention output and MLP output projections zeroed, the residual
  stream is the embedding, so logits reduce to E . rmsnorm(E[t]).
* Sequences in a batch are independent, and physical page placement does not
  change any result (bitwise).
* A step appends exactly one K and one V row per (layer, KV head, sequence),
  at the slot the block table names, holding the bf16 rounding of the step's
  rotated k and raw v; no other byte of the pool changes.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_kv_gqa_qwen3_amd import synth

SHAPE = synth.ModelShape("tiny-test", 2, 128, 4, 2, 32, 192, 512, True)


def _weights(seed=11, shape=SHAPE):
    return synth.make_weights(shape, seed)


def _t(bits):
    return torch.from_numpy(oracle.bf16_to_f64(bits))


def _library_forward(shape, W, tokens):
    """Causal forward over the whole prompt with torch library routines in fp64."""
    H, D, Hq, Hkv = shape.hidden, shape.head_dim, shape.num_q_heads, shape.num_kv_heads
    T = len(tokens)
    eps = shape.rms_eps
    E = _t(W["model.embed_tokens.weight"])
    x = E[torch.as_tensor(tokens, dtype=torch.long)]
    for l in range(shape.num_layers):
        p = f"model.layers.{l}."
        h = F.rms_norm(x, (H,), _t(W[p + "input_layernorm.weight"]), eps=eps)
        q = F.linear(h, _t(W[p + "self_attn.q_proj.weight"])).view(T, Hq, D)
        k = F.linear(h, _t(W[p + "self_attn.k_proj.weight"])).view(T, Hkv, D)
        v = F.linear(h, _t(W[p + "self_attn.v_proj.weight"])).view(T, Hkv, D)
        q = F.rms_norm(q, (D,), _t(W[p + "self_attn.q_norm.weight"]), eps=eps)
        k = F.rms_norm(k, (D,), _t(W[p + "self_attn.k_norm.weight"]), eps=eps)
        q = torch.stack([torch.from_numpy(oracle.rope_neox(q[t].numpy(), t,
                                                           shape.rope_theta))
                         for t in range(T)])
        k = torch.stack([torch.from_numpy(oracle.rope_neox(k[t].numpy(), t,
                                                           shape.rope_theta))
                         for t in range(T)])
        # the pool stores K/V in bf16
        k = torch.from_numpy(oracle.bf16_to_f64(oracle.f64_to_bf16(k.numpy())))
        v = torch.from_numpy(oracle.bf16_to_f64(oracle.f64_to_bf16(v.numpy())))
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True,
                                           enable_gqa=True)[0].transpose(0, 1).reshape(T, -1)
        x = x + F.linear(o, _t(W[p + "self_attn.o_proj.weight"]))
        h2 = F.rms_norm(x, (H,), _t(W[p + "post_attention_layernorm.weight"]), eps=eps)
        a = F.silu(F.linear(h2, _t(W[p + "mlp.gate_proj.weight"]))) * \
            F.linear(h2, _t(W[p + "mlp.up_proj.weight"]))
        x = x + F.linear(a, _t(W[p + "mlp.down_proj.weight"]))
    hf = F.rms_norm(x, (H,), _t(W["model.norm.weight"]), eps=eps)
    head = W["model.embed_tokens.weight"] if shape.tie_embeddings else W["lm_head.weight"]
    return F.linear(hf, _t(head)).numpy()


def _fresh(shape, ctx0, steps, seed, fill=True):
    return synth.make_paged_batch(shape, np.asarray(ctx0), steps, seed, fill_kv=fill)


@pytest.mark.parametrize("tied", [True, False])
def test_stepwise_paged_decode_equals_causal_forward(tied):
    shape = synth.ModelShape("t", 2, 128, 4, 2, 32, 192, 512, tied)
    W = _weights(21, shape)
    T = 37
    prompt = synth.uniform_int(5, "prompt", shape.vocab, T)
    batch = _fresh(shape, [0], T, 3, fill=False)
    orc = oracle.Oracle(shape, W)
    got = []
    for t in range(T):
        lg, nxt, _ = orc.decode_step(prompt[t:t + 1], np.array([t], np.int32),
                                     batch.block_tables, batch.pool)
        got.append(lg[0])
        assert nxt[0] == np.argmax(lg[0])
    got = np.stack(got)
    want = _library_forward(shape, W, prompt)
    scale = np.abs(want).max()
    assert np.abs(got - want).max() <= 1e-10 * scale
    # Oracle.prefill: the last position's logits and greedy id, the same pool
    pool_p = _fresh(shape, [0], T, 3, fill=False).pool
    lg_p, nxt_p = orc.prefill(prompt, batch.block_tables[0], pool_p)
    assert lg_p.shape == (shape.vocab,)
    assert np.abs(lg_p - want[-1]).max() <= 1e-10 * scale
    assert nxt_p == int(np.argmax(want[-1]))
    np.testing.assert_array_equal(pool_p, batch.pool)


@pytest.mark.parametrize("tied", [True, False])
def test_prefill_chunk_equals_causal_forward(tied):
    """Oracle.prefill_chunk with a whole prompt as one chunk (every row a head
    row) gives every position's logits of the library causal forward, and
    fills the pool with the bytes of the one-position-at-a-time loop."""
    shape = synth.ModelShape("t", 2, 128, 4, 2, 32, 192, 512, tied)
    W = _weights(23, shape)
    T = 37
    prompt = synth.uniform_int(6, "prompt", shape.vocab, T)
    batch = _fresh(shape, [0], T, 3, fill=False)
    orc = oracle.Oracle(shape, W)
    tables = np.repeat(batch.block_tables, T, axis=0)
    lg, nxt = orc.prefill_chunk(prompt, np.arange(T, dtype=np.int32), tables, batch.pool, T)
    want = _library_forward(shape, W, prompt)
    scale = np.abs(want).max()
    assert lg.shape == want.shape
    assert np.abs(lg - want).max() <= 1e-10 * scale
    np.testing.assert_array_equal(nxt, np.argmax(want, axis=1))
    pool_s = _fresh(shape, [0], T, 3, fill=False).pool
    orc.prefill(prompt, batch.block_tables[0], pool_s)
    np.testing.assert_array_equal(batch.pool, pool_s)


def test_prefill_chunk_matches_decode_step_rows():
    """A continuation chunk: shuffled rows of two sequences whose earlier
    positions are already in the pool.  prefill_chunk and decode_step (which
    also appends every row before any row attends) agree on the head rows'
    logits to fp64 rounding, on their ids, and on every pool byte; a smaller
    n_head gives the leading rows' logits alone."""
    W = _weights(61)
    orc = oracle.Oracle(SHAPE, W)
    batch = _fresh(SHAPE, [9, 20], 12, 7)
    rows = [(0, 9 + i) for i in range(12)] + [(1, 20 + i) for i in range(7)]
    order = np.random.default_rng(3).permutation(len(rows))
    rows = [rows[i] for i in order]
    tok = synth.uniform_int(8, "chunk", SHAPE.vocab, len(rows))
    pos = np.array([p for _, p in rows], dtype=np.int32)
    tab = batch.block_tables[[s for s, _ in rows]]
    pool_a, pool_b = batch.pool.copy(), batch.pool.copy()
    lg_a, nx_a, _ = orc.decode_step(tok, pos, tab, pool_a)
    lg_b, nx_b = orc.prefill_chunk(tok, pos, tab, pool_b, len(rows))
    assert np.abs(lg_b - lg_a).max() <= 1e-10 * np.abs(lg_a).max()
    np.testing.assert_array_equal(nx_b, nx_a)
    np.testing.assert_array_equal(pool_b, pool_a)
    pool_c = batch.pool.copy()
    lg_c, nx_c = orc.prefill_chunk(tok, pos, tab, pool_c, 3)
    assert lg_c.shape == (3, SHAPE.vocab)
    np.testing.assert_array_equal(lg_c, lg_b[:3])
    np.testing.assert_array_equal(nx_c, nx_b[:3])
    np.testing.assert_array_equal(pool_c, pool_a)


def test_zeroed_blocks_reduce_to_embedding_logits():
    W = _weights(31)
    for l in range(SHAPE.num_layers):
        W[f"model.layers.{l}.self_attn.o_proj.weight"][:] = 0
        W[f"model.layers.{l}.mlp.down_proj.weight"][:] = 0
    batch = _fresh(SHAPE, [5, 19], 1, 4)
    orc = oracle.Oracle(SHAPE, W)
    lg, nxt, _ = orc.decode_step(batch.tokens, batch.positions, batch.block_tables, batch.pool)
    E = _t(W["model.embed_tokens.weight"])
    h = F.rms_norm(E[torch.as_tensor(batch.tokens, dtype=torch.long)], (SHAPE.hidden,),
                   _t(W["model.norm.weight"]), eps=SHAPE.rms_eps)
    want = (h @ E.T).numpy()
    np.testing.assert_allclose(lg, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(nxt, np.argmax(want, axis=1))


def test_batch_sequences_are_independent():
    W = _weights(41)
    orc = oracle.Oracle(SHAPE, W)
    batch = _fresh(SHAPE, [7, 33, 16], 1, 5)
    pool_all = batch.pool.copy()
    lg_all, nx_all, _ = orc.decode_step(batch.tokens, batch.positions, batch.block_tables,
                                        pool_all)
    for b in range(3):
        pool_b = batch.pool.copy()
        lg_b, nx_b, _ = orc.decode_step(batch.tokens[b:b + 1], batch.positions[b:b + 1],
                                        batch.block_tables[b:b + 1], pool_b)
        np.testing.assert_array_equal(lg_b[0], lg_all[b])
        assert nx_b[0] == nx_all[b]


def test_page_placement_does_not_change_results():
    W = _weights(51)
    orc = oracle.Oracle(SHAPE, W)
    a = _fresh(SHAPE, [40, 3], 2, 6)
    b = synth.shuffled_copy(a, 99)
    lg_a, _, _ = orc.decode_step(a.tokens, a.positions, a.block_tables, a.pool)
    lg_b, _, _ = orc.decode_step(b.tokens, b.positions, b.block_tables, b.pool)
    np.testing.assert_array_equal(lg_a, lg_b)


def test_append_writes_exactly_the_expected_slots():
    W = _weights(61)
    orc = oracle.Oracle(SHAPE, W)
    batch = _fresh(SHAPE, [17, 31], 1, 7)
    before = batch.pool.copy()
    _, _, taps0 = orc.decode_step(batch.tokens, batch.positions, batch.block_tables,
                                  batch.pool.copy(), tap_layer=0)
    _, _, taps1 = orc.decode_step(batch.tokens, batch.positions, batch.block_tables,
                                  batch.pool.copy(), tap_layer=1)
    after = batch.pool
    orc.decode_step(batch.tokens, batch.positions, batch.block_tables, after)
    changed = np.zeros(after.shape[:5], dtype=bool)   # per (l, page, kv, head, slot) row
    QD, KD = SHAPE.q_dim, SHAPE.kv_dim
    for l, taps in ((0, taps0), (1, taps1)):
        for b in range(2):
            pos = int(batch.positions[b])
            page = int(batch.block_tables[b, pos // 16])
            for g in range(SHAPE.num_kv_heads):
                changed[l, page, :, g, pos % 16] = True
                np.testing.assert_array_equal(after[l, page, 0, g, pos % 16],
                                              oracle.f64_to_bf16(taps["k_rot"][b, g]))
                v = taps["qkv"][b, QD + KD + g * SHAPE.head_dim:QD + KD + (g + 1) *
                                SHAPE.head_dim]
                np.testing.assert_array_equal(after[l, page, 1, g, pos % 16],
                                              oracle.f64_to_bf16(v))
    np.testing.assert_array_equal(after[~changed], before[~changed])
