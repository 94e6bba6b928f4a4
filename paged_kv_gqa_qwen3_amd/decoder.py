"""Convenience wrapper over the C ABI for Python callers: owns a qd handle and
moves numpy inputs into torch device tensors.  Marshalling only; every step
of the decode path runs in libqd's kernels.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import binding


def _torch():
    import torch  # imported lazily so that CPU-only tools need not load it
    return torch


def to_device_bf16(a: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (same bits)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def to_device_i32(a: np.ndarray, device="cuda"):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def pool_to_device(pool: np.ndarray, device="cuda"):
    """Paged KV pool ([L][P][2][Hkv][16][D] of uint16 bf16 bits, or uint8 E4M3
    codes) -> device int16 (or uint8) tensor."""
    torch = _torch()
    pool = np.ascontiguousarray(pool)
    if pool.dtype == np.uint8:
        return torch.from_numpy(pool).to(device)
    return torch.from_numpy(pool.view(np.int16)).to(device)


def pool_to_host(pool_t) -> np.ndarray:
    a = pool_t.cpu().numpy()
    return a if a.dtype == np.uint8 else a.view(np.uint16)


class Decoder:
    """A qd handle plus the capacity it was created with."""

    def __init__(self, shape, max_batch: int, max_pages_per_seq: int, num_pages: int,
                 use_graphs: bool = True, stream: Optional[int] = None,
                 persistent: bool = False, max_prefill_rows: int = 0, kv_fp8: bool = False,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        torch = _torch()
        self.shape = shape
        self.max_batch = max_batch
        self.max_pages = max_pages_per_seq
        self.num_pages = num_pages
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        self.cfg = binding.make_config(shape, max_batch, max_pages_per_seq, num_pages,
                                       use_graphs, persistent, max_prefill_rows, kv_fp8,
                                       k_scale, v_scale)
        self.handle = binding.qd_create(self.cfg, stream)

    def load_numpy_weights(self, weights: Dict[str, np.ndarray], chunk: int = 24) -> None:
        """Upload HF-named bf16 numpy weights in groups and hand them to the library."""
        torch = _torch()
        names = list(weights)
        for i in range(0, len(names), chunk):
            group = {n: to_device_bf16(weights[n]) for n in names[i:i + chunk]}
            binding.qd_load_weights(self.handle, group)
            del group
        torch.cuda.synchronize()

    def step(self, tokens, positions, tables, pool, next_ids, logits=None) -> None:
        binding.qd_decode_step(self.handle, int(tokens.shape[0]), tokens, positions, tables,
                               pool, next_ids, logits)

    def prefill(self, tokens, positions, tables, pool, n_logits=0, next_ids=None,
                logits=None) -> None:
        """One chunk of prompt rows (qd_prefill): causal across the chunk; rows
        0..n_logits-1 get logits and greedy next ids."""
        binding.qd_prefill(self.handle, int(tokens.shape[0]), tokens, positions, tables, pool,
                           int(n_logits), next_ids, logits)

    def prefill_prompts(self, seq_rows, start_pos, tokens, tables, pool, n_logits=0,
                        next_ids=None, logits=None) -> None:
        """Prompt segments packed back to back (qd_prefill_prompts): segment s
        is seq_rows[s] tokens at positions start_pos[s].. with block-table row
        tables[s]; segments 0..n_logits-1 get their last row's logits and
        greedy next id."""
        binding.qd_prefill_prompts(self.handle, seq_rows, start_pos, tokens, tables, pool,
                                   int(n_logits), next_ids, logits)

    def step_taps(self, tokens, positions, tables, pool, next_ids, logits, taps, layer):
        binding.qd_decode_step_taps(self.handle, int(tokens.shape[0]), tokens, positions,
                                    tables, pool, next_ids, logits, taps, layer)

    def stream_step_taps(self, tokens, positions, tables, pool, next_ids, logits, taps, layer):
        """Batch 1 through the weight-streaming kernel, copying one layer's
        intermediates out (qd_stream_step_taps)."""
        binding.qd_stream_step_taps(self.handle, tokens, positions, tables, pool, next_ids,
                                    logits, taps, layer)

    def sample(self, logits, temperature, top_k, top_p, uniform, out_ids) -> None:
        """Sample each sequence's next token on the device (qd_sample)."""
        binding.qd_sample(self.handle, int(logits.shape[0]), logits, temperature, top_k, top_p,
                          uniform, out_ids)

    def step_path(self, batch: int) -> str:
        """'stream', 'graph' or 'staged': how a step of `batch` runs."""
        return binding.qd_step_path(self.handle, batch)

    def device_status(self) -> int:
        return binding.qd_device_status(self.handle)

    def close(self) -> None:
        if self.handle:
            binding.qd_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
