"""Shared helpers of the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# Logit rule of the decode step (bf16 weights, fp32 accumulation): the largest
# logit difference may be at most 2e-2 of the oracle's largest |logit|.
LOGIT_RTOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_logits(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Element-wise logit bound; returns the observed ratio."""
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU logits"
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    ratio = float((np.abs(gpu - ref) / scale).max())
    assert ratio <= LOGIT_RTOL, f"{what}: max |dlogit| / max|logit| = {ratio:.3e}"
    return ratio


def check_next_ids(gpu_next: np.ndarray, ref_logits: np.ndarray, what: str = "") -> int:
    """Greedy ids must match except where the oracle's top-2 gap is below the
    logit tolerance; a differing id must still be within tolerance of the top."""
    excused = 0
    for b in range(ref_logits.shape[0]):
        row = ref_logits[b]
        tol = LOGIT_RTOL * np.abs(row).max()
        top = int(np.argmax(row))
        if int(gpu_next[b]) == top:
            continue
        top2 = np.sort(row)[-2]
        assert row[top] - top2 < tol, \
            f"{what}: seq {b} next {gpu_next[b]} != {top} with top-2 gap {row[top] - top2:.4f}"
        assert 0 <= gpu_next[b] < row.shape[0]
        assert row[int(gpu_next[b])] >= row[top] - tol, f"{what}: seq {b} picked a far logit"
        excused += 1
    return excused


def gemv_tol(w_bf16: np.ndarray, h: np.ndarray, mfma: bool) -> np.ndarray:
    """Error bound of y = h W^T in fp32 with K-term accumulation: |dy| <=
    (K 2^-24 + d) sum_k |w||h|, d covering the input's own rounding (a bf16
    hi/lo pair, 16 significant bits, on the MFMA path; fp32 normalisation
    otherwise)."""
    N, K = w_bf16.shape
    ha = np.abs(np.atleast_2d(h))
    mag = np.empty((ha.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, 16384):  # row blocks: an LM head's |W| is GBs in fp64
        wa = np.abs(oracle.bf16_to_f64(w_bf16[n0:n0 + 16384]))
        mag[:, n0:n0 + 16384] = ha @ wa.T
    d = 2.0 ** -15 if mfma else 2.0 ** -20
    return (K * 2.0 ** -24 + d) * mag + 1e-30


def bf16_rne_of_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def kv_tol(b):
    """Appended K/V rows (one head_dim row each): bf16 rounding of either side
    (2^-7 relative) plus the projection's own error, which the MFMA path's
    bf16-pair input (about 2^-17 relative per term) can amplify by
    cancellation in small entries: 2^-10 of the row's largest entry."""
    return 2.0 ** -7 * np.abs(b) + 2.0 ** -10 * np.abs(b).max(axis=-1, keepdims=True) + 1e-6


def assert_kv_close(a, b, what=""):
    """a within kv_tol(b) of b; on failure, name the worst entry."""
    tol = kv_tol(b)
    r = np.abs(a - b) / tol
    if not np.all(r <= 1.0):
        i = np.unravel_index(int(np.argmax(r)), r.shape)
        raise AssertionError(f"{what}: KV entry {tuple(int(v) for v in i)} got {a[i]!r} "
                             f"want {b[i]!r} (tol {tol[i]:.3g}); "
                             f"{int((r > 1).sum())} entries out of tolerance")


def appended_mask(batch, pairs):
    """Pool rows (layer, page, K|V, head, slot) written for (sequence, position) pairs."""
    m = np.zeros(batch.pool.shape[:5], dtype=bool)
    for b, p in pairs:
        m[:, batch.block_tables[b, p // 16], :, :, p % 16] = True
    return m
