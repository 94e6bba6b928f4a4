"""Seeded synthetic inputs for the batched decode step.

This module generates inputs only; it holds none of the decode step's
arithmetic.  Both the CPU oracle's tests and the GPU path consume what it
returns, so both sides see identical bytes.

Shapes and distributions follow the workloads the pages measure: Qwen3-4B
(36 layers, hidden 2560, 32 query heads, 8 KV heads, vocabulary 151,936;
"qwen3-runtime" blog, Part 1) decoded at concurrency 1 / 8 / 16 with prompts of
512 / 256 / 256 tokens and at an 8K context (same blog, Part 1 workload table,
workloads A, B, C, E), plus a Qwen3-8B shape (rkmt "从零构建 Qwen3-8B" page,
section 一) and a tiny model for oracle-sized checks.  Weights are N(0, 0.02)
and norm gains 1 + N(0, 0.1), rounded to bf16; cached K/V are N(0, 1) bf16 in
16-token pages (blog Part 4 uses page_size=16) placed by a seeded permutation of
physical pages.  Unused block-table entries point at a NaN-filled poison page,
so a read outside a sequence's context shows up as NaN.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_synth.so")
_lib = None

PAGE = 16
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_void_p, ctypes.c_int64]
        lib.synth_uniform_int.restype = None
        lib.synth_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_int64]
        lib.synth_fill_pool.restype = None
        lib.synth_fill_pool.argtypes = [ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.synth_fill_u16.restype = None
        lib.synth_fill_u16.argtypes = [ctypes.c_void_p, ctypes.c_uint16, ctypes.c_int64]
        lib.synth_fill_pool_fp8.restype = None
        lib.synth_fill_pool_fp8.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.synth_fill_u8.restype = None
        lib.synth_fill_u8.argtypes = [ctypes.c_void_p, ctypes.c_uint8, ctypes.c_int64]
        _lib = lib
    return _lib


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Decoder shape: layers, hidden, query heads, KV heads, head_dim,
    SwiGLU intermediate, vocabulary, tied embeddings, RMSNorm eps, RoPE base."""
    name: str
    num_layers: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tie_embeddings: bool
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def q_dim(self) -> int:
        return self.num_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.num_kv_heads * self.head_dim


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 704, 4096, True)
QWEN3_4B = ModelShape("qwen3-4b", 36, 2560, 32, 8, 128, 9728, 151936, True)
QWEN3_8B = ModelShape("qwen3-8b", 36, 4096, 32, 8, 128, 12288, 151936, False)
SHAPES = {s.name: s for s in (TINY, QWEN3_4B, QWEN3_8B)}


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode workload: model shape, batch, per-sequence context at step 0
    (either fixed or drawn uniformly from [ctx_lo, ctx_hi]) and step count."""
    name: str
    shape: ModelShape
    batch: int
    ctx_lo: int
    ctx_hi: int
    steps: int
    seed: int
    prefill_prompt: int = 0  # >0: context comes from a prompt prefilled by the oracle
    kv_fp8: bool = False     # the KV pool holds E4M3 codes (scales 1) instead of bf16


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny", TINY, 1, 64, 64, 16, 1, prefill_prompt=64),
        Workload("4b_bs1_ctx512", QWEN3_4B, 1, 512, 512, 128, 2),
        Workload("4b_bs8_ctx256", QWEN3_4B, 8, 256, 256, 128, 3),
        Workload("4b_bs16_ctx256", QWEN3_4B, 16, 256, 256, 128, 4),
        Workload("4b_bs1_ctx8192", QWEN3_4B, 1, 8192, 8192, 64, 5),
        Workload("8b_bs8_ragged", QWEN3_8B, 8, 256, 2048, 128, 6),
        Workload("4b_bs8_ctx4096", QWEN3_4B, 8, 4096, 4096, 64, 7),
        Workload("4b_bs8_ctx4096_fp8kv", QWEN3_4B, 8, 4096, 4096, 64, 7, kv_fp8=True),
        # batches beyond the pages' measurements: the 32- and 64-column items
        Workload("4b_bs32_ctx256", QWEN3_4B, 32, 256, 256, 128, 9),
        Workload("4b_bs64_ctx256", QWEN3_4B, 64, 256, 256, 128, 10),
    )
}


def normal_bf16(seed: int, name: str, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(mean, std^2) deviates, keyed by (seed, name)."""
    lib = _load()
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    lib.synth_normal_bf16(lib.synth_key(seed, name.encode()), mean, std,
                          out.ctypes.data, n)
    return out.reshape(shape)


def uniform_int(seed: int, name: str, hi: int, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int32)
    lib.synth_uniform_int(lib.synth_key(seed, name.encode()), hi, out.ctypes.data, n)
    return out


def weight_names(shape: ModelShape) -> List[str]:
    names = ["model.embed_tokens.weight", "model.norm.weight"]
    for l in range(shape.num_layers):
        p = f"model.layers.{l}."
        names += [p + "input_layernorm.weight", p + "self_attn.q_proj.weight",
                  p + "self_attn.k_proj.weight", p + "self_attn.v_proj.weight",
                  p + "self_attn.o_proj.weight", p + "self_attn.q_norm.weight",
                  p + "self_attn.k_norm.weight", p + "post_attention_layernorm.weight",
                  p + "mlp.gate_proj.weight", p + "mlp.up_proj.weight",
                  p + "mlp.down_proj.weight"]
    if not shape.tie_embeddings:
        names.append("lm_head.weight")
    return names


def weight_shape(shape: ModelShape, name: str):
    H, D, I, V = shape.hidden, shape.head_dim, shape.intermediate, shape.vocab
    leaf = name.split(".")[-2] if name.endswith(".weight") else name
    table = {
        "embed_tokens": (V, H), "lm_head": (V, H), "norm": (H,),
        "input_layernorm": (H,), "post_attention_layernorm": (H,),
        "q_proj": (shape.q_dim, H), "k_proj": (shape.kv_dim, H), "v_proj": (shape.kv_dim, H),
        "o_proj": (H, shape.q_dim), "q_norm": (D,), "k_norm": (D,),
        "gate_proj": (I, H), "up_proj": (I, H), "down_proj": (H, I),
    }
    return table[leaf]


def is_norm(name: str) -> bool:
    return name.endswith("norm.weight") or name.endswith("layernorm.weight")


def make_weights(shape: ModelShape, seed: int,
                 names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """Seeded bf16 weights (uint16 bit patterns), HF naming and [out, in] layout.
    Matrices ~ N(0, 0.02); every norm gain ~ 1 + N(0, 0.1)."""
    out = {}
    for name in (names or weight_names(shape)):
        if is_norm(name):
            out[name] = normal_bf16(seed, name, weight_shape(shape, name), 1.0, 0.1)
        else:
            out[name] = normal_bf16(seed, name, weight_shape(shape, name), 0.0, 0.02)
    return out


@dataclasses.dataclass
class PagedBatch:
    """Paged KV pool plus the per-sequence metadata for the first decode step.

    pool          uint16 [L][num_pages][2][Hkv][16][D]  (bf16 bit patterns), or
                  uint8 (E4M3 codes) for an 8-bit pool
    block_tables  int32  [B][max_pages]  physical page ids (poison for unused)
    positions     int32  [B]  position of the token decoded at step 0 (= ctx0)
    tokens        int32  [B]  token decoded at step 0
    """
    pool: np.ndarray
    block_tables: np.ndarray
    positions: np.ndarray
    tokens: np.ndarray
    num_pages: int
    max_pages: int
    poison_page: int


def context_lengths(w: Workload) -> np.ndarray:
    if w.ctx_lo == w.ctx_hi:
        return np.full(w.batch, w.ctx_lo, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + 17))
    return rng.integers(w.ctx_lo, w.ctx_hi + 1, size=w.batch).astype(np.int32)


def make_paged_batch(shape: ModelShape, ctx0: np.ndarray, steps: int, seed: int,
                     fill_kv: bool = True, spare_pages: int = 0,
                     kv_fp8: bool = False) -> PagedBatch:
    """Allocate a pool holding every page the batch touches over `steps` decode
    steps, give each sequence its pages from one seeded permutation of the
    physical page ids (consecutive slices of it), fill the first ctx0[b] slots
    of each sequence with N(0,1) bf16 K/V (with kv_fp8: an 8-bit pool of
    random E4M3 codes, magnitudes 2^-4 .. 3.75), and poison one extra page
    with NaN."""
    ctx0 = np.asarray(ctx0, dtype=np.int32)
    B = len(ctx0)
    need = [-(-(int(c) + steps) // PAGE) for c in ctx0]
    max_pages = max(need)
    num_pages = sum(need) + 1 + spare_pages
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + 29))
    perm = rng.permutation(num_pages).astype(np.int32)
    poison = int(perm[-1])
    tables = np.full((B, max_pages), poison, dtype=np.int32)
    off = 0
    for b in range(B):
        tables[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    L, Hkv, D = shape.num_layers, shape.num_kv_heads, shape.head_dim
    pool = np.zeros((L, num_pages, 2, Hkv, PAGE, D), dtype=np.uint8 if kv_fp8 else np.uint16)
    lib = _load()
    # the poison page is NaN in every layer, K and V
    for l in range(L):
        sl = pool[l, poison]
        if kv_fp8:
            lib.synth_fill_u8(sl.ctypes.data, E4M3_NAN, sl.size)
        else:
            lib.synth_fill_u16(sl.ctypes.data, BF16_NAN, sl.size)
    if fill_kv and int(ctx0.max()) > 0:
        key = lib.synth_key(seed, b"kv_context")
        if kv_fp8:
            lib.synth_fill_pool_fp8(key, pool.ctypes.data, L, num_pages, Hkv, PAGE, D, B,
                                    ctx0.ctypes.data, tables.ctypes.data, max_pages,
                                    int(ctx0.max()))
        else:
            lib.synth_fill_pool(key, 1.0, pool.ctypes.data, L, num_pages, Hkv, PAGE, D, B,
                                ctx0.ctypes.data, tables.ctypes.data, max_pages,
                                int(ctx0.max()))
    tokens = uniform_int(seed, "first_tokens", shape.vocab, B)
    return PagedBatch(pool, tables, ctx0.copy(), tokens, num_pages, max_pages, poison)


def shuffled_copy(batch: PagedBatch, seed: int) -> PagedBatch:
    """The same logical K/V under a different physical placement: pages are
    renumbered by a seeded permutation and moved accordingly."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = batch.num_pages
    newid = rng.permutation(P).astype(np.int32)  # old page p -> newid[p]
    pool = np.empty_like(batch.pool)
    pool[:, newid] = batch.pool
    tables = newid[batch.block_tables]
    return PagedBatch(pool, tables, batch.positions.copy(), batch.tokens.copy(),
                      P, batch.max_pages, int(newid[batch.poison_page]))
