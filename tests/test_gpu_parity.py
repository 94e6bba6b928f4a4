"""GPU parity: libqd's decode step against the CPU oracle, through the C ABI.

* Teacher-forced multi-step runs (both sides receive the oracle's token, each
  keeps its own pool): logits within 2e-2 of max|logit|, greedy ids equal
  unless the oracle's top-2 gap is within that tolerance.
* Stage isolation through the library's taps: every stage of one layer is
  recomputed by the oracle from the GPU's own input to that stage, so each
  kernel is checked against its own error bound; the KV append must be
  bit-exact (placement and rounding) and touch nothing else.
* Graph replay equals eager launches bitwise; physical page placement does
  not change any bit; two identical steps give identical bits.
* Full-size shapes (Qwen3-4B batch 1/8/16, 8K context; Qwen3-8B ragged
  batch 8) in the launch configuration the benchmark times (captured graph).
"""
import gc

import numpy as np
import pytest

import oracle
from paged_kv_gqa_qwen3_amd import binding, synth
from paged_kv_gqa_qwen3_amd.decoder import Decoder, pool_to_device, pool_to_host
from gpu_util import (LOGIT_RTOL, appended_mask as _appended_mask,
                      assert_kv_close as _assert_kv_close, bf16_rne_of_f32, check_logits,
                      check_next_ids, gemv_tol, kv_tol as _kv_tol, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return _t


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class StepIO:
    """Static device buffers for repeated steps (so that graphs replay)."""

    def __init__(self, torch, B, max_pages, V, logits=True):
        self.torch = torch
        self.tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.pos = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.tab = torch.zeros(B, max_pages, dtype=torch.int32, device="cuda")
        self.nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros(B, V, dtype=torch.float32, device="cuda") if logits else None

    def set(self, tokens, positions, tables):
        t = self.torch
        self.tok.copy_(t.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.pos.copy_(t.from_numpy(np.asarray(positions, dtype=np.int32)))
        self.tab.copy_(t.from_numpy(np.asarray(tables, dtype=np.int32)))

    def run(self, dec, pool):
        dec.step(self.tok, self.pos, self.tab, pool, self.nxt, self.logits)


# ----------------------------------------------------------------------------- tiny workload

@pytest.mark.parametrize("persistent", [False, True], ids=["graph", "persistent"])
def test_tiny_workload_teacher_forced(torch, persistent):
    """Tiny GQA decoder: oracle prefill of 64 random tokens, then 16 greedy
    decode steps on the GPU (graph replay, or on a persistent handle the
    weight-streaming kernel), teacher-forced by the oracle."""
    w = synth.WORKLOADS["tiny"]
    shape = w.shape
    W = synth.make_weights(shape, w.seed)
    orc = oracle.Oracle(shape, W)
    batch = synth.make_paged_batch(shape, [0], w.prefill_prompt + w.steps, w.seed, fill_kv=False)
    prompt = synth.uniform_int(w.seed, "prompt", shape.vocab, w.prefill_prompt)
    pool_or = batch.pool
    _, token = orc.prefill(prompt, batch.block_tables[0], pool_or)
    pool_start = pool_or.copy()
    pool = pool_to_device(pool_or)
    dec = Decoder(shape, 1, batch.max_pages, batch.num_pages, persistent=persistent)
    dec.load_numpy_weights(W)
    io = StepIO(torch, 1, batch.max_pages, shape.vocab)
    pos = w.prefill_prompt
    worst = 0.0
    for step in range(w.steps):
        say(f"tiny step {step} pos {pos}")
        io.set([token], [pos], batch.block_tables)
        io.run(dec, pool)
        lg_or, nx_or, _ = orc.decode_step(np.array([token], np.int32), np.array([pos], np.int32),
                                          batch.block_tables, pool_or)
        torch.cuda.synchronize()
        worst = max(worst, check_logits(io.logits.cpu().numpy(), lg_or, f"step {step}"))
        check_next_ids(io.nxt.cpu().numpy(), lg_or, f"step {step}")
        token = int(nx_or[0])
        pos += 1
    assert dec.device_status() == 0
    say(f"tiny worst logit ratio {worst:.3e}")
    got = pool_to_host(pool)
    m = _appended_mask(batch, [(0, q) for q in range(w.prefill_prompt, pos)])
    np.testing.assert_array_equal(got[~m], pool_start[~m])
    a, b = oracle.bf16_to_f64(got[m]), oracle.bf16_to_f64(pool_or[m])
    _assert_kv_close(a, b, "appended KV")
    dec.close()


# ----------------------------------------------------------------------------- stage isolation

def _stage_checks(shape, W, batch, taps, pool_before, pool_after, layer, logits, nxt, mfma,
                  kv=oracle.BF16):
    B = batch.tokens.shape[0]
    H, D, Hq, Hkv = shape.hidden, shape.head_dim, shape.num_q_heads, shape.num_kv_heads
    QD, KD = shape.q_dim, shape.kv_dim
    eps = shape.rms_eps
    pos = batch.positions
    p = f"model.layers.{layer}."
    t = {k: v.astype(np.float64) for k, v in taps.items()}

    if layer == 0:  # the embedding gather: exactly the tokens' bf16 rows
        np.testing.assert_array_equal(
            t["x_in"], oracle.bf16_to_f64(W["model.embed_tokens.weight"][batch.tokens]))

    # RMSNorm + fused QKV projection, from the GPU's residual
    h = oracle.rmsnorm(t["x_in"], W[p + "input_layernorm.weight"], eps)
    Wqkv = np.concatenate([W[p + "self_attn.q_proj.weight"], W[p + "self_attn.k_proj.weight"],
                           W[p + "self_attn.v_proj.weight"]])
    want = oracle.linear(h, Wqkv)
    assert np.all(np.abs(t["qkv"] - want) <= gemv_tol(Wqkv, h, mfma)), "qkv"

    # q/k RMSNorm + NeoX RoPE, from the GPU's projections
    for b in range(B):
        q = t["qkv"][b, :QD].reshape(Hq, D)
        k = t["qkv"][b, QD:QD + KD].reshape(Hkv, D)
        qr = oracle.rope_neox(oracle.rmsnorm(q, W[p + "self_attn.q_norm.weight"], eps), pos[b],
                              shape.rope_theta)
        kr = oracle.rope_neox(oracle.rmsnorm(k, W[p + "self_attn.k_norm.weight"], eps), pos[b],
                              shape.rope_theta)
        assert np.abs(t["q_rot"][b] - qr).max() <= 2e-5 * max(1.0, np.abs(qr).max()), "q_rot"
        assert np.abs(t["k_rot"][b] - kr).max() <= 2e-5 * max(1.0, np.abs(kr).max()), "k_rot"

    # KV append: bit-exact rounding and placement.  An 8-bit pool stores the
    # E4M3 code of value / scale; the tests' scales are powers of two, so the
    # fp32 product the kernel encodes is exact and the oracle's encoding of
    # the same value is the same decision.
    def rounded(x, scale):
        if kv.fp8:
            return oracle.f64_to_e4m3(x.astype(np.float64) / scale)
        return bf16_rne_of_f32(x)
    for b in range(B):
        page = batch.block_tables[b, pos[b] // 16]
        slot = pos[b] % 16
        np.testing.assert_array_equal(pool_after[layer, page, 0, :, slot],
                                      rounded(taps["k_rot"][b], kv.k_scale))
        v = taps["qkv"][b, QD + KD:].reshape(Hkv, D)
        np.testing.assert_array_equal(pool_after[layer, page, 1, :, slot],
                                      rounded(v, kv.v_scale))
    m = _appended_mask(batch, list(enumerate(pos)))
    np.testing.assert_array_equal(pool_after[~m], pool_before[~m])

    # paged GQA attention, from the GPU's rotated q and the pool after the append
    for b in range(B):
        o = oracle.attention(t["q_rot"][b], pool_after, layer, batch.block_tables[b],
                             int(pos[b]) + 1, Hkv, kv)
        vmax = np.abs(oracle.pool_values(pool_after, kv)[layer][:, 1]).max()
        vmax = vmax if np.isfinite(vmax) else 10.0
        assert np.abs(t["attn"][b] - o).max() <= 2e-4 * max(1.0, vmax), f"attn seq {b}"

    # O projection + residual
    a = t["attn"].reshape(B, QD)
    Wo = W[p + "self_attn.o_proj.weight"]
    want = t["x_in"] + oracle.linear(a, Wo)
    tol = gemv_tol(Wo, a, mfma) + 2.0 ** -22 * np.abs(want)
    assert np.all(np.abs(t["x_mid"] - want) <= tol), "x_mid"

    # RMSNorm + gate/up projection + SwiGLU
    h2 = oracle.rmsnorm(t["x_mid"], W[p + "post_attention_layernorm.weight"], eps)
    Wg, Wu = W[p + "mlp.gate_proj.weight"], W[p + "mlp.up_proj.weight"]
    g, u = oracle.linear(h2, Wg), oracle.linear(h2, Wu)
    want = oracle.silu(g) * u
    tg, tu = gemv_tol(Wg, h2, mfma), gemv_tol(Wu, h2, mfma)
    tol = 1.1 * np.abs(u) * tg + np.abs(oracle.silu(g)) * tu + tg * tu + 1e-6 * np.abs(want)
    assert np.all(np.abs(t["act"] - want) <= tol), "act"

    # down projection + residual
    Wd = W[p + "mlp.down_proj.weight"]
    want = t["x_mid"] + oracle.linear(t["act"], Wd)
    tol = gemv_tol(Wd, t["act"], mfma) + 2.0 ** -22 * np.abs(want)
    assert np.all(np.abs(t["x_out"] - want) <= tol), "x_out"

    if layer == shape.num_layers - 1:
        hf = oracle.rmsnorm(t["x_out"], W["model.norm.weight"], eps)
        assert np.abs(t["final_h"] - hf).max() <= 1e-5 * max(1.0, np.abs(hf).max()), "final_h"
        E = W["model.embed_tokens.weight"] if shape.tie_embeddings else W["lm_head.weight"]
        want = oracle.linear(t["final_h"], E)
        assert np.all(np.abs(logits - want) <= gemv_tol(E, t["final_h"], mfma) * 1.01 + 1e-6), \
            "logits"
        # the on-device argmax is exact on the GPU's own logits (lowest index on ties)
        np.testing.assert_array_equal(nxt, np.argmax(logits, axis=1))


def _run_stage_checks(torch, shape, W, batch, what, stream=False, kv=oracle.BF16):
    """One step through a taps entry point, stopping at the first and last
    layer, each stage checked by the oracle from the GPU's own input to it:
    the per-stage kernels (no graph), or with stream=True the batch-1
    weight-streaming kernel (MFMA tiles on a bf16 pair of the input).  kv:
    the pool's element type (an 8-bit pool for kv.fp8)."""
    B = batch.tokens.shape[0]
    mfma = B > 1 or stream
    dec = Decoder(shape, B, batch.max_pages, batch.num_pages, use_graphs=False,
                  persistent=stream, kv_fp8=kv.fp8, k_scale=kv.k_scale, v_scale=kv.v_scale)
    if stream:
        assert B == 1 and dec.step_path(1) == "stream"
    dec.load_numpy_weights(W)
    QD, KD = shape.q_dim, shape.kv_dim
    for layer in (0, shape.num_layers - 1):
        say(f"stages {what} layer={layer}")
        pool = pool_to_device(batch.pool)
        taps = {
            "x_in": torch.zeros(B, shape.hidden, device="cuda"),
            "qkv": torch.zeros(B, QD + 2 * KD, device="cuda"),
            "q_rot": torch.zeros(B, shape.num_q_heads, shape.head_dim, device="cuda"),
            "k_rot": torch.zeros(B, shape.num_kv_heads, shape.head_dim, device="cuda"),
            "attn": torch.zeros(B, shape.num_q_heads, shape.head_dim, device="cuda"),
            "x_mid": torch.zeros(B, shape.hidden, device="cuda"),
            "act": torch.zeros(B, shape.intermediate, device="cuda"),
            "x_out": torch.zeros(B, shape.hidden, device="cuda"),
            "final_h": torch.zeros(B, shape.hidden, device="cuda"),
        }
        logits = torch.zeros(B, shape.vocab, device="cuda")
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        run = dec.stream_step_taps if stream else dec.step_taps
        run(_i32(torch, batch.tokens), _i32(torch, batch.positions),
            _i32(torch, batch.block_tables), pool, nxt, logits, taps, layer)
        torch.cuda.synchronize()
        tp = {k: v.cpu().numpy() for k, v in taps.items()}
        _stage_checks(shape, W, batch, tp, batch.pool, pool_to_host(pool), layer,
                      logits.cpu().numpy(), nxt.cpu().numpy(), mfma, kv)
    assert dec.device_status() == 0
    dec.close()


@pytest.mark.parametrize("B,ctx", [
    (1, [0]), (1, [15]), (1, [16]), (2, [17, 300]), (3, [31, 32, 33]), (4, [1, 64, 129, 200]),
    (5, [0, 15, 16, 100, 255]), (8, [3] * 8), (16, list(range(0, 320, 20))),
    # splits of 8 pages (batch <= 8, at most 128 pages per sequence) or 24
    # pages: one to 17 of them, a combine of more than 16 splits (2100), and
    # of 20 (7600: the combine that loads every split's partials in one round
    # trip, up to 24 splits)
    (3, [511, 512, 1100]), (6, [0, 511, 512, 1100, 40, 2000]), (1, [2100]), (1, [7600]),
    # 32- and 64-column MFMA items, up to the largest batch a handle takes
    (24, [(37 * i) % 400 for i in range(24)]), (33, [(53 * i) % 300 for i in range(33)]),
    (64, [(29 * i) % 200 for i in range(64)]),
])
def test_tiny_stages(torch, B, ctx):
    shape = synth.TINY
    W = synth.make_weights(shape, 100 + B)
    batch = synth.make_paged_batch(shape, ctx, 1, 200 + B)
    _run_stage_checks(torch, shape, W, batch, f"B={B} ctx={ctx}")


def _two_layers(base):
    return synth.ModelShape(base.name + "-2l", 2, base.hidden, base.num_q_heads,
                            base.num_kv_heads, base.head_dim, base.intermediate, base.vocab,
                            base.tie_embeddings)


WIDE = {"4b": synth.QWEN3_4B, "8b": synth.QWEN3_8B}


@pytest.mark.parametrize("model", list(WIDE))
def test_wide_items_stages(torch, model):
    """Qwen3-4B and -8B widths (2 layers) at batch 16, stage by stage: at 16
    batch columns gate/up (both widths) and down (8B) take items of 128 rows
    (two row tiles per wave, one input operand read for both), which the
    tiny shapes are too small to use (too few items for the CUs)."""
    shape = _two_layers(WIDE[model])
    W = _weights(shape, 5)
    ctx = [(97 * i) % 600 for i in range(16)]
    batch = synth.make_paged_batch(shape, ctx, 1, 250)
    _run_stage_checks(torch, shape, W, batch, f"{shape.name} B=16")


@pytest.mark.parametrize("model,B", [("4b", 24), ("4b", 64), ("8b", 40)])
def test_wide_batch_stages(torch, model, B):
    """Qwen3-4B and -8B widths (2 layers) at 24, 40 and 64 batch columns,
    stage by stage: items of 128 rows that stream their input slice through
    LDS in chunks of 4 k-tiles, a K split only to give half the CUs an item,
    and the splits of a row group summing one share of its outputs each
    (1 to 7 splits; down at K = 9728 and 12288: 11 and 24 chunks per item,
    8B QKV slices of 43 k-tiles ending in a partial chunk).  The tiny
    shapes reach these items too, with one k-tile per split."""
    shape = _two_layers(WIDE[model])
    W = _weights(shape, 6)
    ctx = [(61 * i) % 500 for i in range(B)]
    batch = synth.make_paged_batch(shape, ctx, 1, 252 + B)
    _run_stage_checks(torch, shape, W, batch, f"{shape.name} B={B}")


@pytest.mark.parametrize("model", list(WIDE))
def test_wide_items_fused_matches_staged(torch, model):
    """The same 128-row items inside the fused MLP launch (qd_decode_step,
    graph) and as per-stage launches (qd_decode_step_taps) at Qwen3-4B and
    -8B widths, batch 16: the same logits, ids and pool bits.  (The fused
    launch sizes its LDS for both item kinds; a 64-row size would cut off
    the end of a 128-row item's input slice.)"""
    shape = _two_layers(WIDE[model])
    W = _weights(shape, 5)
    ctx = [(53 * i) % 500 for i in range(16)]
    batch = synth.make_paged_batch(shape, ctx, 1, 251)
    dec = Decoder(shape, 16, batch.max_pages, batch.num_pages, use_graphs=True)
    dec.load_numpy_weights(W)
    pf, ps = pool_to_device(batch.pool), pool_to_device(batch.pool)
    a = StepIO(torch, 16, batch.max_pages, shape.vocab)
    b = StepIO(torch, 16, batch.max_pages, shape.vocab)
    for io in (a, b):
        io.set(batch.tokens, batch.positions, batch.block_tables)
    a.run(dec, pf)
    dec.step_taps(b.tok, b.pos, b.tab, ps, b.nxt, b.logits, None, -1)
    torch.cuda.synchronize()
    assert torch.equal(a.logits, b.logits) and torch.equal(a.nxt, b.nxt)
    assert torch.equal(pf, ps)
    assert dec.device_status() == 0
    dec.close()


# Every (head_dim, query heads per KV head) pair the attention kernel is
# built for, on small models (2 layers, hidden 256, 2 KV heads), at batch 1
# (the fp32-input GEMV items) and batch 5 (MFMA items), with one split, a
# few and a combine over more than 16.
@pytest.mark.parametrize("D,G", [(64, 1), (64, 2), (64, 4), (128, 1), (128, 2), (128, 4)])
@pytest.mark.parametrize("ctx", [[700], [0, 17, 300, 40, 1100]], ids=["b1", "b5"])
def test_head_shapes_stages(torch, D, G, ctx):
    shape = synth.ModelShape(f"d{D}g{G}", 2, 256, 2 * G, 2, D, 704, 4096, True)
    seed = 300 + D + G
    W = synth.make_weights(shape, seed)
    batch = synth.make_paged_batch(shape, ctx, 1, seed)
    _run_stage_checks(torch, shape, W, batch, f"D={D} G={G} ctx={ctx}")


# An 8-bit (E4M3) pool: the append's codes bit-exact, attention over the
# codes times their scales, every other stage unchanged; batch 1 (VALU
# GEMV), 5 and 16 (MFMA items), one split up to a combine of more than 16,
# head_dim 64 and 128.  The scales are powers of two (0.5 for K, 2 for V).
@pytest.mark.parametrize("shape_name", ["d64g2", "d128g4"])
@pytest.mark.parametrize("ctx", [[0], [700], [0, 17, 300, 40, 1100], list(range(0, 320, 20))],
                         ids=["b1", "b1_700", "b5", "b16"])
def test_fp8_pool_stages(torch, shape_name, ctx):
    shape = synth.TINY if shape_name == "d64g2" else \
        synth.ModelShape("d128g4", 2, 256, 8, 2, 128, 704, 4096, True)
    seed = 400 + len(ctx) + shape.head_dim
    W = synth.make_weights(shape, seed)
    batch = synth.make_paged_batch(shape, ctx, 1, seed, kv_fp8=True)
    _run_stage_checks(torch, shape, W, batch, f"fp8 {shape_name} ctx={ctx}",
                      kv=oracle.KvFormat(True, 0.5, 2.0))


@pytest.mark.parametrize("persistent", [False, True], ids=["graph", "persistent"])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.25, 3.0)], ids=["unit", "scaled"])
def test_fp8_pool_teacher_forced(torch, persistent, scales):
    """Decode steps on an 8-bit pool (batches 1 and 3; a persistent handle
    runs batch 1 through the per-stage graph, the streaming kernel taking
    bf16 pools only), each side keeping its own pool, ids teacher-forced by
    the oracle; logits to the decode step's bound at every step."""
    shape = synth.TINY
    kv = oracle.KvFormat(True, *scales)
    W = synth.make_weights(shape, 501)
    orc = oracle.Oracle(shape, W)
    for ctx in ([40], [5, 70, 300]):
        B = len(ctx)
        batch = synth.make_paged_batch(shape, ctx, 8, 502 + B, kv_fp8=True)
        dec = Decoder(shape, B, batch.max_pages, batch.num_pages, persistent=persistent,
                      kv_fp8=True, k_scale=kv.k_scale, v_scale=kv.v_scale)
        assert dec.step_path(B) == "graph"
        dec.load_numpy_weights(W)
        pool = pool_to_device(batch.pool)
        pool_or = batch.pool.copy()
        io = StepIO(torch, B, batch.max_pages, shape.vocab)
        tokens, positions = batch.tokens.copy(), batch.positions.copy()
        for step in range(8):
            say(f"fp8 teacher-forced B={B} persistent={persistent} step {step}")
            io.set(tokens, positions, batch.block_tables)
            io.run(dec, pool)
            lg_or, nx_or, _ = orc.decode_step(tokens, positions, batch.block_tables, pool_or,
                                              kv=kv)
            torch.cuda.synchronize()
            check_logits(io.logits.cpu().numpy(), lg_or, f"fp8 B={B} step {step}")
            check_next_ids(io.nxt.cpu().numpy(), lg_or, f"fp8 B={B} step {step}")
            tokens, positions = nx_or.astype(np.int32), positions + 1
        assert dec.device_status() == 0
        dec.close()


def test_max_context_stages(torch):
    """The longest block-table row a handle takes (2048 pages, 32768 tokens):
    the step at position 32767, a combine over 86 splits of 24 pages."""
    shape = synth.TINY
    W = synth.make_weights(shape, 91)
    batch = synth.make_paged_batch(shape, [32767], 1, 92)
    assert batch.max_pages == 2048
    _run_stage_checks(torch, shape, W, batch, "ctx=32767")


@pytest.mark.parametrize("ctx", [[0], [15], [16], [40], [700], [2047]])
def test_tiny_stream_stages(torch, ctx):
    """The batch-1 weight-streaming kernel, stage by stage (its taps entry
    point): one split, several, and the longest context a streaming handle
    takes (128 pages, a combine over 32 splits)."""
    shape = synth.TINY
    W = synth.make_weights(shape, 400 + ctx[0] % 13)
    batch = synth.make_paged_batch(shape, ctx, 1, 401 + ctx[0] % 7)
    _run_stage_checks(torch, shape, W, batch, f"stream ctx={ctx}", stream=True)


def test_full_size_stream_stages(torch):
    """The headline's kernel at the Qwen3-4B shape, context 512, stage by
    stage at the first and the last layer (the LM head and argmax included)."""
    w = synth.WORKLOADS["4b_bs1_ctx512"]
    shape = w.shape
    W = _weights(shape, 2)
    batch = synth.make_paged_batch(shape, synth.context_lengths(w), 2, w.seed)
    _run_stage_checks(torch, shape, W, batch, "stream 4b ctx=512", stream=True)
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- invariances

def test_graph_replay_matches_eager(torch):
    shape = synth.TINY
    W = synth.make_weights(shape, 7)
    batch = synth.make_paged_batch(shape, [5, 40, 77], 6, 8)
    dg = Decoder(shape, 4, batch.max_pages, batch.num_pages, use_graphs=True)
    de = Decoder(shape, 4, batch.max_pages, batch.num_pages, use_graphs=False)
    dg.load_numpy_weights(W)
    de.load_numpy_weights(W)
    pg, pe = pool_to_device(batch.pool), pool_to_device(batch.pool)
    ig = StepIO(torch, 3, batch.max_pages, shape.vocab)
    ie = StepIO(torch, 3, batch.max_pages, shape.vocab)
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    for step in range(6):
        say(f"graph vs eager step {step}")
        ig.set(tokens, positions, batch.block_tables)
        ie.set(tokens, positions, batch.block_tables)
        ig.run(dg, pg)
        ie.run(de, pe)
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # unrelated eager work
        assert torch.equal(ig.logits, ie.logits)
        assert torch.equal(ig.nxt, ie.nxt)
        tokens = ie.nxt.cpu().numpy()
        positions = positions + 1
    assert torch.equal(pg, pe)
    dg.close()
    de.close()


@pytest.mark.parametrize("B,ctx", [(3, [5, 40, 77]), (4, [0, 16, 250, 31]), (2, [700, 1300])])
def test_persistent_handle_mixed_batches(torch, B, ctx):
    """A persistent handle runs batch 1 as the streaming kernel and larger
    batches as the per-stage graph, sharing its scratch between the two.
    Steps of both sizes interleaved on one handle must give the same bits as
    the same steps on a graph-only handle (batch B) and on a batch-1
    streaming handle (the first sequence alone, on a pool of its own)."""
    shape = synth.TINY
    W = synth.make_weights(shape, 70 + B)
    batch = synth.make_paged_batch(shape, ctx, 5, 71 + B)
    mp, npg = batch.max_pages, batch.num_pages
    dp = Decoder(shape, B, mp, npg, persistent=True)
    dg = Decoder(shape, B, mp, npg, persistent=False)
    ds = Decoder(shape, 1, mp, npg, persistent=True)
    assert [dp.step_path(b) for b in (1, B)] == ["stream", "graph"]
    assert ds.step_path(1) == "stream"
    for d in (dp, dg, ds):
        d.load_numpy_weights(W)
    pools = [pool_to_device(batch.pool) for _ in range(4)]  # dp batch B, dg, dp batch 1, ds
    io = [StepIO(torch, B, mp, shape.vocab), StepIO(torch, B, mp, shape.vocab),
          StepIO(torch, 1, mp, shape.vocab), StepIO(torch, 1, mp, shape.vocab)]
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    tok1, pos1 = batch.tokens[:1].copy(), batch.positions[:1].copy()
    for step in range(5):
        say(f"mixed batches B={B} step {step}")
        for i, d in ((0, dp), (2, dp), (1, dg), (3, ds)):
            if i < 2:
                io[i].set(tokens, positions, batch.block_tables)
            else:
                io[i].set(tok1, pos1, batch.block_tables[:1])
            io[i].run(d, pools[i])
        torch.cuda.synchronize()
        assert torch.equal(io[0].logits, io[1].logits)
        assert torch.equal(io[0].nxt, io[1].nxt)
        assert torch.equal(io[2].logits, io[3].logits)
        assert torch.equal(io[2].nxt, io[3].nxt)
        tokens, positions = io[1].nxt.cpu().numpy(), positions + 1
        tok1, pos1 = io[3].nxt.cpu().numpy(), pos1 + 1
    assert torch.equal(pools[0], pools[1])
    assert torch.equal(pools[2], pools[3])
    for d in (dp, dg, ds):
        assert d.device_status() == 0
        d.close()


@pytest.mark.parametrize("ctx", [[40], [700], [2000], [0]])
def test_stream_step_matches_staged(torch, ctx):
    """Batch 1 on a persistent handle runs the weight-streaming kernel (MFMA
    tiles against a bf16 pair of the input); the per-stage kernels of the
    same handle (VALU, fp32 input) must agree within the logit tolerance
    over chained steps, greedy ids must agree unless near a tie, and the KV
    rows both append must agree to bf16 rounding.  Short, split and long
    contexts (one split, several, the combine over more than 16 splits: the
    longest a streaming handle takes, 128 pages); a repeated step must give
    the same bits."""
    shape = synth.TINY
    W = synth.make_weights(shape, 80 + ctx[0] % 7)
    batch = synth.make_paged_batch(shape, ctx, 5, 81)
    dp = Decoder(shape, 1, batch.max_pages, batch.num_pages, persistent=True)
    assert dp.step_path(1) == "stream", batch.max_pages
    dp.load_numpy_weights(W)
    pp, pe = pool_to_device(batch.pool), pool_to_device(batch.pool)
    ip = StepIO(torch, 1, batch.max_pages, shape.vocab)
    ie = StepIO(torch, 1, batch.max_pages, shape.vocab)
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    for step in range(5):
        say(f"stream vs staged ctx={ctx} step {step}")
        ip.set(tokens, positions, batch.block_tables)
        ie.set(tokens, positions, batch.block_tables)
        ip.run(dp, pp)
        torch.cuda.synchronize()
        first = ip.logits.clone()
        if step == 0:  # the same step again (it rewrites the same KV slot)
            ip.run(dp, pp)
            torch.cuda.synchronize()
            assert torch.equal(first, ip.logits)
        dp.step_taps(ie.tok, ie.pos, ie.tab, pe, ie.nxt, ie.logits, None, -1)
        torch.cuda.synchronize()
        ref = ie.logits.cpu().numpy().astype(np.float64)
        check_logits(ip.logits.cpu().numpy(), ref, f"step {step}")
        check_next_ids(ip.nxt.cpu().numpy(), ref, f"step {step}")
        tokens = ie.nxt.cpu().numpy()
        positions = positions + 1
    got, want = pool_to_host(pp), pool_to_host(pe)
    m = _appended_mask(batch, [(0, int(batch.positions[0]) + q) for q in range(5)])
    np.testing.assert_array_equal(got[~m], want[~m])
    _assert_kv_close(oracle.bf16_to_f64(got[m]), oracle.bf16_to_f64(want[m]),
                     "stream vs staged appended KV")
    assert dp.device_status() == 0
    dp.close()


def test_profiling_entry_points(torch):
    """qd_profile_step runs the step as the per-stage kernels, the same items
    and split plans as qd_decode_step (whose MLP half is one fused launch
    at this batch): the same logits, ids and pool bits; it reports a
    positive time for every class it launched; qd_profile_class times one
    projection class alone and leaves the next step's results unchanged."""
    shape = synth.TINY
    W = synth.make_weights(shape, 55)
    batch = synth.make_paged_batch(shape, [5, 40, 77], 2, 56)
    B = 3
    dp = Decoder(shape, B, batch.max_pages, batch.num_pages, use_graphs=False)
    dp.load_numpy_weights(W)
    pa, pb = pool_to_device(batch.pool), pool_to_device(batch.pool)
    ia = StepIO(torch, B, batch.max_pages, shape.vocab)
    ib = StepIO(torch, B, batch.max_pages, shape.vocab)
    for io in (ia, ib):
        io.set(batch.tokens, batch.positions, batch.block_tables)
    ia.run(dp, pa)
    prof = binding.qd_profile_step(dp.handle, B, ib.tok, ib.pos, ib.tab, pb, ib.nxt, ib.logits)
    torch.cuda.synchronize()
    assert torch.equal(ia.logits, ib.logits) and torch.equal(ia.nxt, ib.nxt)
    assert torch.equal(pa, pb)
    for cls, (ms, n) in prof.items():
        assert n >= 1 and ms > 0.0, (cls, ms, n)
    for cls in ("qkv", "o_proj", "gate_up", "down", "lm_head"):
        us = binding.qd_profile_class(dp.handle, B, cls, reps=3)
        assert us > 0.0, cls
    with pytest.raises(binding.QdError):
        binding.qd_profile_class(dp.handle, B, "attention", reps=3)
    ib.tok.copy_(ia.tok)  # the classes overwrote only scratch: the next step is unchanged
    pb.copy_(pa)
    ia.run(dp, pa)
    ib.run(dp, pb)
    torch.cuda.synchronize()
    assert torch.equal(ia.logits, ib.logits)
    assert dp.device_status() == 0
    dp.close()


@pytest.mark.parametrize("shape_name,B,ctx", [
    ("tiny", 1, [37]), ("tiny", 3, [5, 40, 300]), ("tiny", 8, [0, 16, 31, 100, 255, 256, 700, 2]),
    ("tiny", 16, [(41 * i) % 900 for i in range(16)]), ("tiny", 17, [(13 * i) % 200 for i in range(17)]),
    ("d128g4", 5, [3, 17, 200, 513, 64]), ("d128g4", 1, [2000]),
])
def test_fused_step_matches_per_stage(torch, shape_name, B, ctx):
    """At batches 2-16 qd_decode_step runs the MLP half of every layer as one
    launch (gate/up items, then down items that wait on completion
    counters) with alternating residual buffer sets; the items and split
    plans are the per-stage kernels', so over chained steps the logits,
    ids and the whole pool must equal the per-stage path's
    (qd_decode_step_taps) bit for bit.  Batches 1 and 17 take the
    per-stage launches either way."""
    shape = synth.TINY if shape_name == "tiny" else \
        synth.ModelShape("d128g4", 2, 256, 8, 2, 128, 704, 4096, True)
    W = synth.make_weights(shape, 600 + B)
    batch = synth.make_paged_batch(shape, ctx, 4, 601 + B)
    dec = Decoder(shape, B, batch.max_pages, batch.num_pages, use_graphs=True)
    dec.load_numpy_weights(W)
    pf, pe = pool_to_device(batch.pool), pool_to_device(batch.pool)
    io_f = StepIO(torch, B, batch.max_pages, shape.vocab)
    io_e = StepIO(torch, B, batch.max_pages, shape.vocab)
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    for step in range(4):
        say(f"fused vs per-stage {shape_name} B={B} step {step}")
        io_f.set(tokens, positions, batch.block_tables)
        io_e.set(tokens, positions, batch.block_tables)
        io_f.run(dec, pf)
        dec.step_taps(io_e.tok, io_e.pos, io_e.tab, pe, io_e.nxt, io_e.logits, None, -1)
        torch.cuda.synchronize()
        assert torch.isfinite(io_f.logits).all()
        assert torch.equal(io_f.logits, io_e.logits), step
        assert torch.equal(io_f.nxt, io_e.nxt), step
        tokens, positions = io_e.nxt.cpu().numpy(), positions + 1
    torch.cuda.synchronize()
    assert torch.equal(pf, pe)
    assert dec.device_status() == 0
    dec.close()


def test_step_paths(torch):
    """qd_step_path: a persistent handle streams batch 1 only when sized for
    at most 128 pages per sequence and runs every larger batch as the graph;
    a non-persistent handle always takes the graph; batches outside
    1..max_batch are rejected."""
    shape = synth.TINY
    for pages, persistent, want in ((128, True, ["stream"] + ["graph"] * 5),
                                    (129, True, ["graph"] * 6),
                                    (16, False, ["graph"] * 6)):
        dec = Decoder(shape, 6, pages, pages + 1, persistent=persistent)
        assert [dec.step_path(b) for b in range(1, 7)] == want, (pages, persistent)
        for bad in (0, 7):
            with pytest.raises(binding.QdError):
                dec.step_path(bad)
        dec.close()


def test_page_placement_and_determinism(torch):
    shape = synth.TINY
    W = synth.make_weights(shape, 9)
    a = synth.make_paged_batch(shape, [100, 3, 47, 250, 16], 1, 10)
    b = synth.shuffled_copy(a, 11)
    dec = Decoder(shape, 5, a.max_pages, a.num_pages, use_graphs=False)
    dec.load_numpy_weights(W)
    outs = []
    for bt in (a, a, b):
        pool = pool_to_device(bt.pool)
        io = StepIO(torch, 5, bt.max_pages, shape.vocab)
        io.set(bt.tokens, bt.positions, bt.block_tables)
        io.run(dec, pool)
        torch.cuda.synchronize()
        outs.append((io.logits.cpu().numpy(), io.nxt.cpu().numpy(), pool_to_host(pool)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][2], outs[1][2])
    np.testing.assert_array_equal(outs[0][0], outs[2][0])
    np.testing.assert_array_equal(outs[0][1], outs[2][1])


def test_bad_device_inputs_are_flagged_not_faulting(torch):
    shape = synth.TINY
    W = synth.make_weights(shape, 12)
    batch = synth.make_paged_batch(shape, [10, 20, 30], 1, 13)
    dec = Decoder(shape, 3, batch.max_pages, batch.num_pages, use_graphs=False)
    dec.load_numpy_weights(W)
    from paged_kv_gqa_qwen3_amd import binding
    cases = [
        ("token", dict(tokens=[shape.vocab + 5, 1, 2]), binding.QD_DEV_BAD_TOKEN),
        ("position", dict(positions=[10, batch.max_pages * 16 + 3, 30]),
         binding.QD_DEV_BAD_POSITION),
        ("page", dict(page=(2, 0, batch.num_pages + 7)), binding.QD_DEV_BAD_PAGE),
    ]
    for name, case, bit in cases:
        say(f"bad input: {name}")
        tokens = np.array(case.get("tokens", batch.tokens), np.int32)
        positions = np.array(case.get("positions", batch.positions), np.int32)
        tables = batch.block_tables.copy()
        if "page" in case:
            r, c, v = case["page"]
            tables[r, c] = v
        pool = pool_to_device(batch.pool)
        io = StepIO(torch, 3, batch.max_pages, shape.vocab)
        io.set(tokens, positions, tables)
        io.run(dec, pool)
        assert dec.device_status() & bit
    assert dec.device_status() == 0


# ----------------------------------------------------------------------------- full size

_WEIGHTS = {}


def _weights(shape, seed):
    key = (shape.name, seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        gc.collect()
        say(f"generating {shape.name} weights (seed {seed})")
        _WEIGHTS[key] = synth.make_weights(shape, seed)
    return _WEIGHTS[key]


# Every workload through the per-stage graph; the one that a persistent
# handle runs differently (batch 1 at a short context: the streaming kernel)
# also on such a handle.
@pytest.mark.parametrize("name,persistent", [
    (n, False) for n in ("4b_bs1_ctx512", "4b_bs8_ctx256", "4b_bs16_ctx256", "4b_bs1_ctx8192",
                         "8b_bs8_ragged", "4b_bs8_ctx4096", "4b_bs8_ctx4096_fp8kv",
                         "4b_bs32_ctx256")] +
    [("4b_bs1_ctx512", True)],
    ids=lambda v: v if isinstance(v, str) else ("persistent" if v else "graph"))
def test_full_size_steps(torch, name, persistent):
    w = synth.WORKLOADS[name]
    shape = w.shape
    W = _weights(shape, 2 if shape is synth.QWEN3_4B else w.seed)
    ctx0 = synth.context_lengths(w)
    kv = oracle.KvFormat(True) if w.kv_fp8 else oracle.BF16
    batch = synth.make_paged_batch(shape, ctx0, w.steps, w.seed, kv_fp8=w.kv_fp8)
    say(f"{name} persistent={persistent}: B={w.batch} ctx0={ctx0.tolist()} "
        f"pages={batch.num_pages}")
    orc = oracle.Oracle(shape, W)
    dec = Decoder(shape, w.batch, batch.max_pages, batch.num_pages, use_graphs=True,
                  persistent=persistent, kv_fp8=w.kv_fp8)
    assert dec.step_path(w.batch) == ("stream" if persistent else "graph")
    dec.load_numpy_weights(W)
    pool = pool_to_device(batch.pool)
    pool_or = batch.pool
    io = StepIO(torch, w.batch, batch.max_pages, shape.vocab)
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    for step in range(2):
        say(f"{name}: step {step}")
        io.set(tokens, positions, batch.block_tables)
        io.run(dec, pool)
        lg_or, nx_or, _ = orc.decode_step(tokens, positions, batch.block_tables, pool_or,
                                          kv=kv)
        torch.cuda.synchronize()
        r = check_logits(io.logits.cpu().numpy(), lg_or, f"{name} step {step}")
        ex = check_next_ids(io.nxt.cpu().numpy(), lg_or, f"{name} step {step}")
        say(f"{name}: step {step} logit ratio {r:.3e}, excused ids {ex}")
        tokens, positions = nx_or.astype(np.int32), positions + 1
    assert dec.device_status() == 0
    dec.close()
    del pool
    torch.cuda.empty_cache()


def test_prefix_shared_pages_match_private_copies(torch):
    """Sequences built with the page manager: A prefilled (by the oracle) and
    its 48-token prompt prefix published; B takes those three pages from the
    prefix cache and prefills only its own suffix; C holds B's tokens in
    pages of its own.  Decode steps of [A, B, C] on the GPU give B and C the
    same bits, and leave the shared pages untouched."""
    shape = synth.TINY
    W = synth.make_weights(shape, 41)
    orc = oracle.Oracle(shape, W)
    rng = np.random.default_rng(42)
    prefix = rng.integers(0, shape.vocab, 48).astype(np.int32)
    pa = np.concatenate([prefix, rng.integers(0, shape.vocab, 10).astype(np.int32)])
    pb = np.concatenate([prefix, rng.integers(0, shape.vocab, 7).astype(np.int32)])
    steps, max_pages, num_pages = 4, 8, 24
    pad = num_pages  # an extra page, never used, as the table filler
    L, Hkv, D = shape.num_layers, shape.num_kv_heads, shape.head_dim
    pool = np.zeros((L, num_pages + 1, 2, Hkv, 16, D), dtype=np.uint16)
    mgr = binding.PageManager(num_pages, max_pages)
    mgr.add(0)
    mgr.reserve(0, len(pa) + steps)
    row_a = mgr.tables([0], pad)[0]
    _, tok_a = orc.prefill(pa, row_a, pool)
    assert mgr.publish(0, pa) == 3
    mgr.add(1)
    assert mgr.match(1, pb) == 48
    mgr.reserve(1, len(pb) + steps)
    mgr.add(2)
    mgr.reserve(2, len(pb) + steps)
    rows = mgr.tables([0, 1, 2], pad)
    assert list(rows[1][:3]) == list(row_a[:3]) and not set(rows[2]) & set(row_a[:3])
    for t in range(48, len(pb)):  # B: only its suffix
        orc.decode_step(pb[t:t + 1], np.array([t], np.int32), rows[1:2], pool, want_logits=False)
    _, tok_c = orc.prefill(pb, rows[2], pool)
    shared = [int(p) for p in row_a[:3]]
    before = pool[:, shared].copy()
    dec = Decoder(shape, 3, max_pages, num_pages + 1)
    dec.load_numpy_weights(W)
    dpool = pool_to_device(pool)
    io = StepIO(torch, 3, max_pages, shape.vocab)
    tokens = np.array([tok_a, tok_c, tok_c], np.int32)
    positions = np.array([len(pa), len(pb), len(pb)], np.int32)
    for step in range(steps):
        say(f"prefix sharing step {step}")
        io.set(tokens, positions, rows)
        io.run(dec, dpool)
        torch.cuda.synchronize()
        assert torch.equal(io.logits[1], io.logits[2]), step
        assert torch.equal(io.nxt[1], io.nxt[2]), step
        tokens = io.nxt.cpu().numpy()
        tokens[2] = tokens[1]
        positions = positions + 1
    np.testing.assert_array_equal(pool_to_host(dpool)[:, shared], before)
    assert dec.device_status() == 0
    dec.close()
    mgr.close()


def test_forked_sequence_matches_its_source(torch):
    """A sequence forked by the page manager (full pages shared, the partly
    filled page copied on the device) decodes the same tokens to the same
    bits as its source, and diverging tokens leave the shared pages as they
    were."""
    shape = synth.TINY
    W = synth.make_weights(shape, 43)
    orc = oracle.Oracle(shape, W)
    prompt = np.random.default_rng(44).integers(0, shape.vocab, 40).astype(np.int32)
    steps, max_pages, num_pages = 3, 6, 16
    L, Hkv, D = shape.num_layers, shape.num_kv_heads, shape.head_dim
    pool = np.zeros((L, num_pages + 1, 2, Hkv, 16, D), dtype=np.uint16)
    mgr = binding.PageManager(num_pages, max_pages)
    mgr.add(0)
    mgr.reserve(0, len(prompt))
    _, tok = orc.prefill(prompt, mgr.tables([0], num_pages)[0], pool)
    cs, cd = mgr.fork(0, 1)
    assert cs >= 0 and cd >= 0
    for s in (0, 1):
        mgr.reserve(s, len(prompt) + steps)
    rows = mgr.tables([0, 1], num_pages)
    shared = [int(p) for p in rows[0][:2]]
    assert list(rows[1][:2]) == shared
    dpool = pool_to_device(pool)
    dpool[:, cd] = dpool[:, cs]  # the device copy the fork asks for
    before = pool_to_host(dpool)[:, shared].copy()
    dec = Decoder(shape, 2, max_pages, num_pages + 1)
    dec.load_numpy_weights(W)
    io = StepIO(torch, 2, max_pages, shape.vocab)
    io.set([tok, tok], [len(prompt)] * 2, rows)
    io.run(dec, dpool)
    torch.cuda.synchronize()
    assert torch.equal(io.logits[0], io.logits[1])
    nxt = io.nxt.cpu().numpy()
    io.set([nxt[0], (nxt[0] + 1) % shape.vocab], [len(prompt) + 1] * 2, rows)
    io.run(dec, dpool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool_to_host(dpool)[:, shared], before)
    assert dec.device_status() == 0
    dec.close()
    mgr.close()


# ----------------------------------------------------------------------------- prefill

def _prefill_chunks(prompts, chunk, seed):
    """The prompts' (sequence, position) rows in chunks of `chunk`, positions
    in order across chunks (so a chunk's earlier positions are in the pool),
    sequences interleaved; in each chunk the rows holding a prompt's last
    token come first (they get logits), the others in a seeded random order.
    Returns [(rows, n_logits)]."""
    rng = np.random.default_rng(seed)
    rows = sorted((p, s) for s, pr in enumerate(prompts) for p in range(len(pr)))
    out = []
    for i in range(0, len(rows), chunk):
        c = [(s, p) for p, s in rows[i:i + chunk]]
        last = [r for r in c if r[1] == len(prompts[r[0]]) - 1]
        rest = [r for r in c if r[1] != len(prompts[r[0]]) - 1]
        order = rng.permutation(len(rest))
        out.append((last + [rest[j] for j in order], len(last)))
    return out


def _check_prefill(torch, shape, W, prompts, chunk, persistent, seed):
    """GPU chunked prefill (qd_prefill) against the oracle running each prompt
    one position at a time: the last position's logits and greedy id, every
    appended K/V row, and no other pool row touched."""
    V = shape.vocab
    batch = synth.make_paged_batch(shape, [0] * len(prompts), max(len(p) for p in prompts),
                                   seed, fill_kv=False)
    tables = batch.block_tables
    pool_start = batch.pool.copy()
    pool = pool_to_device(batch.pool)
    dec = Decoder(shape, chunk, batch.max_pages, batch.num_pages, persistent=persistent)
    dec.load_numpy_weights(W)
    got = {}
    for ci, (rows, n) in enumerate(_prefill_chunks(prompts, chunk, seed)):
        say(f"prefill {shape.name} chunk {ci}: {len(rows)} rows, {n} with logits")
        tok = _i32(torch, [prompts[s][p] for s, p in rows])
        pos = _i32(torch, [p for _, p in rows])
        tab = _i32(torch, tables[[s for s, _ in rows]])
        nxt = torch.full((max(n, 1),), -1, dtype=torch.int32, device="cuda")
        lg = torch.zeros(max(n, 1), V, dtype=torch.float32, device="cuda")
        dec.prefill(tok, pos, tab, pool, n, nxt if n else None, lg if n else None)
        torch.cuda.synchronize()
        for i in range(n):
            got[rows[i][0]] = (lg[i].cpu().numpy(), nxt[i:i + 1].cpu().numpy())
    assert dec.device_status() == 0
    dec.close()
    orc = oracle.Oracle(shape, W)
    pool_or = batch.pool
    for s, pr in enumerate(prompts):
        say(f"prefill {shape.name}: oracle, prompt {s} ({len(pr)} tokens)")
        lg_or, _ = orc.prefill(pr, tables[s], pool_or)
        r = check_logits(got[s][0][None], lg_or[None], f"prompt {s}")
        check_next_ids(got[s][1], lg_or[None], f"prompt {s}")
        say(f"prefill prompt {s}: logit ratio {r:.3e}")
    host = pool_to_host(pool)
    m = _appended_mask(batch, [(s, p) for s, pr in enumerate(prompts) for p in range(len(pr))])
    np.testing.assert_array_equal(host[~m], pool_start[~m])
    # Layer 0's K/V come from the embedding through one projection: the
    # one-stage bound of the decode step's append.  Deeper layers' K/V are
    # outputs of the whole stack below them, like the logits, and take the
    # logits' end-to-end bound (LOGIT_RTOL of the row's largest magnitude)
    # plus either side's bf16 rounding.
    _assert_kv_close(oracle.bf16_to_f64(host[0][m[0]]), oracle.bf16_to_f64(pool_or[0][m[0]]),
                     "prefill KV, layer 0")
    worst = 0.0
    for l in range(1, shape.num_layers):
        a, b = oracle.bf16_to_f64(host[l][m[l]]), oracle.bf16_to_f64(pool_or[l][m[l]])
        scale = np.abs(b).max(axis=-1, keepdims=True) + 1e-30
        r = np.abs(a - b) / (2.0 ** -7 * np.abs(b) + LOGIT_RTOL * scale)
        worst = max(worst, float(r.max()))
        assert np.all(r <= 1.0), f"prefill KV, layer {l}: worst ratio {float(r.max()):.3f}"
    say(f"prefill KV: worst end-to-end ratio {worst:.3f} (layers 1..{shape.num_layers - 1})")


@pytest.mark.parametrize("lens,chunk,persistent", [
    ([70, 45], 24, False),      # rows from two prompts, one logit row per ending chunk
    ([33, 33, 20], 64, False),  # a 64-row chunk, then two prompts ending in one chunk
    ([17, 9], 8, True),         # persistent handle: prefill still runs the staged kernels
    ([1], 1, True),             # one-token prompt: the batch-1 kernels
])
def test_tiny_prefill_matches_oracle(torch, lens, chunk, persistent):
    shape = synth.TINY
    seed = 300 + sum(lens) + chunk
    W = synth.make_weights(shape, seed)
    prompts = [synth.uniform_int(seed + i, "prompt", shape.vocab, n) for i, n in enumerate(lens)]
    _check_prefill(torch, shape, W, prompts, chunk, persistent, seed)


def test_full_size_prefill_matches_oracle(torch):
    """Qwen3-4B shape: two prompts (20 and 12 tokens) in 16-row chunks; the
    second chunk ends both prompts (logits for two rows)."""
    shape = synth.QWEN3_4B
    W = _weights(shape, 2)
    prompts = [synth.uniform_int(500 + i, "prompt", shape.vocab, n) for i, n in enumerate([20, 12])]
    _check_prefill(torch, shape, W, prompts, 16, False, 5)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("persistent", [False, True], ids=["graph", "persistent"])
def test_prefill_then_decode_end_to_end(torch, persistent):
    """The whole request on the GPU: a 40-token prompt prefilled in 16-row
    chunks (qd_prefill), then 8 greedy decode steps from the prefill's own
    next id, each teacher-forced by the oracle (which prefills one position
    at a time), logits and ids checked at every step."""
    shape = synth.TINY
    W = synth.make_weights(shape, 77)
    n, steps = 40, 8
    prompt = synth.uniform_int(77, "prompt", shape.vocab, n)
    batch = synth.make_paged_batch(shape, [0], n + steps, 77, fill_kv=False)
    table = batch.block_tables
    pool = pool_to_device(batch.pool)
    pool_or = batch.pool.copy()
    dec = Decoder(shape, 16, batch.max_pages, batch.num_pages, persistent=persistent)
    dec.load_numpy_weights(W)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
    for c0 in range(0, n, 16):
        pos = list(range(c0, min(c0 + 16, n)))
        last = pos[-1] == n - 1
        if last:
            pos = [pos[-1]] + pos[:-1]
        dec.prefill(_i32(torch, prompt[pos]), _i32(torch, pos), _i32(torch, table[[0] * len(pos)]),
                    pool, 1 if last else 0, nxt if last else None, lg if last else None)
    orc = oracle.Oracle(shape, W)
    lg_or, token = orc.prefill(prompt, table[0], pool_or)
    torch.cuda.synchronize()
    check_logits(lg.cpu().numpy(), lg_or[None], "prefill")
    check_next_ids(nxt.cpu().numpy(), lg_or[None], "prefill")
    io = StepIO(torch, 1, batch.max_pages, shape.vocab)
    for step in range(steps):
        say(f"prefill+decode persistent={persistent} step {step}")
        io.set([token], [n + step], table)
        io.run(dec, pool)
        lg_or, nx_or, _ = orc.decode_step(np.array([token], np.int32),
                                          np.array([n + step], np.int32), table, pool_or)
        torch.cuda.synchronize()
        check_logits(io.logits.cpu().numpy(), lg_or, f"step {step}")
        check_next_ids(io.nxt.cpu().numpy(), lg_or, f"step {step}")
        token = int(nx_or[0])
    assert dec.device_status() == 0
    dec.close()


def test_prefill_rejects_bad_arguments(torch):
    """Argument errors come back as codes and launch nothing: rows outside
    1..max_batch, n_logits outside 0..rows, no next-id output while logits
    are asked for, weights not loaded."""
    shape = synth.TINY
    batch = synth.make_paged_batch(shape, [0], 32, 3, fill_kv=False)
    dec = Decoder(shape, 4, batch.max_pages, batch.num_pages)
    pool = pool_to_device(batch.pool)
    tok, pos = _i32(torch, [1, 2, 3, 4]), _i32(torch, [0, 1, 2, 3])
    tab = _i32(torch, np.repeat(batch.block_tables, 4, axis=0))
    nxt = torch.zeros(4, dtype=torch.int32, device="cuda")
    h = dec.handle
    with pytest.raises(binding.QdError):  # weights not loaded
        binding.qd_prefill(h, 4, tok, pos, tab, pool, 1, nxt)
    dec.load_numpy_weights(synth.make_weights(shape, 3))
    for rows, n, out in ((0, 0, nxt), (5, 1, nxt), (4, 5, nxt), (4, -1, nxt), (4, 1, None)):
        with pytest.raises(binding.QdError):
            binding.qd_prefill(h, rows, tok, pos, tab, pool, n, out)
    binding.qd_prefill(h, 4, tok, pos, tab, pool, 0)  # a chunk without logits is fine
    torch.cuda.synchronize()
    assert dec.device_status() == 0
    dec.close()
