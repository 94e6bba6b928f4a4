"""Algorithmic HBM bytes and FLOPs of one batched decode step.

A decode step must read every weight once (shared by the whole batch; the
pages' point that decode GEMV runs at about 1 FLOP per byte and batching raises
it, "推理引擎里面发生了什么", Decode section) and every cached K/V byte of
each sequence once; it writes one K and one V row per layer and KV head for
each sequence.  Everything else (activations, partial sums) stays on chip or
in cache and is not counted.
"""
from __future__ import annotations

from typing import Iterable

BF16 = 2


def linear_weight_bytes(shape) -> int:
    """Bytes of the per-layer projections summed over layers (bf16)."""
    H, I = shape.hidden, shape.intermediate
    qkv = (shape.q_dim + 2 * shape.kv_dim) * H
    o = H * shape.q_dim
    gate_up = 2 * I * H
    down = H * I
    return shape.num_layers * (qkv + o + gate_up + down) * BF16


def lm_head_bytes(shape) -> int:
    return shape.vocab * shape.hidden * BF16


def norm_bytes(shape) -> int:
    per_layer = 2 * shape.hidden + 2 * shape.head_dim
    return (shape.num_layers * per_layer + shape.hidden) * BF16


def weight_bytes_per_step(shape) -> int:
    """All weights a step reads once: projections, LM head, norm gains."""
    return linear_weight_bytes(shape) + lm_head_bytes(shape) + norm_bytes(shape)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int = BF16) -> int:
    """K and V bytes one token occupies across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def step_bytes(shape, ctx: Iterable[int], kv_elem_bytes: int = BF16) -> int:
    """Algorithmic HBM bytes of one step whose sequences attend ctx[b] tokens
    (ctx[b] = position + 1, the appended token included): weights once, the
    embedding rows of the batch, and ctx[b] K/V rows per sequence (ctx-1 read,
    1 written) of kv_elem_bytes per element (2 for bf16, 1 for an 8-bit
    pool)."""
    ctx = list(ctx)
    kv = kv_bytes_per_token(shape.num_layers, shape.num_kv_heads, shape.head_dim, kv_elem_bytes)
    return (weight_bytes_per_step(shape) + len(ctx) * shape.hidden * BF16 +
            sum(int(c) for c in ctx) * kv)


def step_flops(shape, ctx: Iterable[int]) -> int:
    """Multiply-adds x 2 of the projections and attention for one step."""
    ctx = list(ctx)
    B = len(ctx)
    per_tok = (linear_weight_bytes(shape) + lm_head_bytes(shape)) // BF16 * 2
    attn = sum(4 * shape.num_q_heads * shape.head_dim * int(c) * shape.num_layers
               for c in ctx)
    return B * per_tok + attn


def gemm_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k
