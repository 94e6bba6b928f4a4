"""The seeded input generator: deterministic, the stated distributions, and
page placement that keeps every logical token's content."""
import numpy as np

import oracle
from paged_kv_gqa_qwen3_amd import synth


def test_deterministic_and_keyed_by_name():
    a = synth.normal_bf16(3, "x", (1000,))
    b = synth.normal_bf16(3, "x", (1000,))
    c = synth.normal_bf16(3, "y", (1000,))
    np.testing.assert_array_equal(a, b)
    assert (a != c).mean() > 0.9


def test_distributions():
    w = oracle.bf16_to_f64(synth.normal_bf16(5, "w", (400_000,), 0.0, 0.02))
    assert abs(w.mean()) < 2e-4 and abs(w.std() - 0.02) < 2e-4
    g = oracle.bf16_to_f64(synth.normal_bf16(5, "g", (400_000,), 1.0, 0.1))
    assert abs(g.mean() - 1.0) < 2e-3 and abs(g.std() - 0.1) < 1e-3
    ids = synth.uniform_int(5, "ids", 151936, 200_000)
    assert ids.min() >= 0 and ids.max() < 151936 and abs(ids.mean() / 151936 - 0.5) < 0.01


def test_paged_batch_layout_and_shuffle():
    shape = synth.TINY
    b = synth.make_paged_batch(shape, np.array([40, 17]), 5, 9)
    assert b.pool.shape == (2, b.num_pages, 2, 2, 16, 64)
    # every page of a sequence is distinct, and no page is shared
    used = [p for row in b.block_tables for p in row if p != b.poison_page]
    assert len(used) == len(set(used)) == b.num_pages - 1
    assert np.isnan(oracle.bf16_to_f64(b.pool[:, b.poison_page])).all()
    s = synth.shuffled_copy(b, 4)
    for seq in range(2):
        for t in range(int(b.positions[seq])):
            pa = b.block_tables[seq, t // 16]
            pb = s.block_tables[seq, t // 16]
            np.testing.assert_array_equal(b.pool[:, pa, :, :, t % 16],
                                          s.pool[:, pb, :, :, t % 16])
