"""CPU oracle for the batched Qwen3-style GQA decode step.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the GPU library never does.  It
shares no code with the GPU path.  The arithmetic lives in ``qd_oracle.c``
(plain loops, fp64 throughout; only the weights and the KV pool are bf16, as
the pages fix, or the pool is OCP E4M3 with per-tensor K and V scales for the
FP8 variant); this module marshals numpy arrays into it.

Every function here is pinned by tests under ``tests/`` against closed forms,
invariants, library routines or brute force (see the test module docstrings).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_oracle.so")
_lib = None

PAGE = 16


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int), ("hidden", ctypes.c_int),
                ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("intermediate", ctypes.c_int),
                ("vocab", ctypes.c_int), ("tie_embeddings", ctypes.c_int),
                ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


_P = ctypes.c_void_p


class _Layer(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("in_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm",
                                  "post_norm", "wgate", "wup", "wdown")]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("lm_head", _P),
                ("layers", ctypes.POINTER(_Layer))]


class _Kv(ctypes.Structure):
    _fields_ = [("fp8", ctypes.c_int), ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double)]


class KvFormat:
    """Element type of a KV pool: bf16 (the default), or OCP E4M3 ("fp8")
    with one scale for K and one for V (stored code = E4M3(value / scale))."""

    def __init__(self, fp8: bool = False, k_scale: float = 1.0, v_scale: float = 1.0):
        self.fp8, self.k_scale, self.v_scale = bool(fp8), float(k_scale), float(v_scale)

    def _c(self):
        return _Kv(int(self.fp8), self.k_scale, self.v_scale)

    @property
    def dtype(self):
        return np.uint8 if self.fp8 else np.uint16


BF16 = KvFormat()


class _Taps(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int)] + [
        (n, _P) for n in ("x_in", "qkv", "q_rot", "k_rot", "attn", "x_mid", "act", "x_out",
                          "final_h")]


TAP_NAMES = ("x_in", "qkv", "q_rot", "k_rot", "attn", "x_mid", "act", "x_out", "final_h")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.or_bf16_to_f64.restype = ctypes.c_double
        lib.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f64_to_bf16.restype = ctypes.c_uint16
        lib.or_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.or_rmsnorm.restype = None
        lib.or_rmsnorm.argtypes = [_P, ctypes.c_int, _P, ctypes.c_double, _P]
        lib.or_linear.restype = None
        lib.or_linear.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P]
        lib.or_rope_neox.restype = None
        lib.or_rope_neox.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.or_attention.restype = None
        lib.or_attention.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P,
                                     ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P,
                                     ctypes.POINTER(_Kv)]
        lib.or_e4m3_to_f64.restype = ctypes.c_double
        lib.or_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.or_f64_to_e4m3.restype = ctypes.c_uint8
        lib.or_f64_to_e4m3.argtypes = [ctypes.c_double]
        lib.or_f64_to_e4m3_n.restype = None
        lib.or_f64_to_e4m3_n.argtypes = [_P, ctypes.c_int64, _P]
        lib.or_e4m3_to_f64_n.restype = None
        lib.or_e4m3_to_f64_n.argtypes = [_P, ctypes.c_int64, _P]
        lib.or_silu.restype = ctypes.c_double
        lib.or_silu.argtypes = [ctypes.c_double]
        lib.or_f64_to_bf16_n.restype = None
        lib.or_f64_to_bf16_n.argtypes = [_P, ctypes.c_int64, _P]
        lib.or_silu_n.restype = None
        lib.or_silu_n.argtypes = [_P, ctypes.c_int64, _P]
        lib.or_argmax.restype = ctypes.c_int
        lib.or_argmax.argtypes = [_P, ctypes.c_int]
        lib.or_decode_step.restype = ctypes.c_int
        lib.or_decode_step.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights),
                                       ctypes.c_int, _P, _P, _P, ctypes.c_int, _P,
                                       ctypes.c_int, _P, _P, ctypes.POINTER(_Taps),
                                       ctypes.POINTER(_Kv)]
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _req(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"expected C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


# ----------------------------------------------------------------------------- scalar ops

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 bit pattern (ties to even), one rounding step."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.or_f64_to_bf16_n(x.ctypes.data, x.size, out.ctypes.data)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP E4M3 codes -> exact float64 values (NaN for 0x7F / 0xFF)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib.or_e4m3_to_f64_n(c.ctypes.data, c.size, out.ctypes.data)
    return out


def f64_to_e4m3(x) -> np.ndarray:
    """float64 -> nearest E4M3 code (ties to even, saturating at +-448)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.or_f64_to_e4m3_n(x.ctypes.data, x.size, out.ctypes.data)
    return out


def pool_values(pool, kv: "KvFormat" = BF16) -> np.ndarray:
    """The values a pool [L][P][2][Hkv][16][D] holds, as float64."""
    if not kv.fp8:
        return bf16_to_f64(pool)
    v = e4m3_to_f64(pool)
    v[:, :, 0] *= kv.k_scale
    v[:, :, 1] *= kv.v_scale
    return v


def rmsnorm(x, gain_bf16, eps: float = 1e-6) -> np.ndarray:
    lib = _load()
    x = _f64(x)
    g = _req(gain_bf16, np.uint16)
    n = x.shape[-1]
    assert g.shape == (n,)
    y = np.empty_like(x)
    xf, yf = x.reshape(-1, n), y.reshape(-1, n)
    for r in range(xf.shape[0]):
        lib.or_rmsnorm(xf[r].ctypes.data, n, g.ctypes.data, eps, yf[r].ctypes.data)
    return y


def linear(x, w_bf16) -> np.ndarray:
    """x [B, K] float64, w [N, K] bf16 -> [B, N]."""
    lib = _load()
    x = _f64(np.atleast_2d(x))
    w = _req(w_bf16, np.uint16)
    B, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    y = np.empty((B, N), dtype=np.float64)
    lib.or_linear(x.ctypes.data, B, K, w.ctypes.data, N, y.ctypes.data)
    return y


def rope_neox(v, pos: int, theta: float = 1e6) -> np.ndarray:
    """NeoX rotary embedding of each row of v (last axis = head_dim) at pos."""
    lib = _load()
    v = _f64(v).copy()
    D = v.shape[-1]
    vf = v.reshape(-1, D)
    for r in range(vf.shape[0]):
        lib.or_rope_neox(vf[r].ctypes.data, D, int(pos), theta)
    return v


def attention(q, pool, layer: int, table_row, ctx: int, num_kv_heads: int,
              kv: "KvFormat" = BF16) -> np.ndarray:
    """q [Hq, D] float64; pool [L][P][2][Hkv][16][D] of kv's type; -> o [Hq, D]."""
    lib = _load()
    q = _f64(q)
    pool = _req(pool, kv.dtype)
    row = _req(np.asarray(table_row, dtype=np.int32), np.int32)
    Hq, D = q.shape
    assert pool.shape[3] == num_kv_heads and pool.shape[5] == D and pool.shape[4] == PAGE
    assert len(row) * PAGE >= ctx
    o = np.empty_like(q)
    ckv = kv._c()
    lib.or_attention(q.ctypes.data, Hq, num_kv_heads, D, pool.ctypes.data, pool.shape[1],
                     layer, row.ctypes.data, ctx, o.ctypes.data, ctypes.byref(ckv))
    return o


def silu(z) -> np.ndarray:
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.empty(z.shape, dtype=np.float64)
    lib.or_silu_n(z.ctypes.data, z.size, out.ctypes.data)
    return out


def argmax(v) -> int:
    lib = _load()
    v = _f64(v)
    return int(lib.or_argmax(v.ctypes.data, v.shape[0]))


# ----------------------------------------------------------------------------- decode step

class Oracle:
    """Holds a model's bf16 weights (HF names) and runs decode steps on a pool."""

    def __init__(self, shape, weights: Dict[str, np.ndarray]):
        self.shape = shape
        self._weights = weights
        self._keep = []
        c = _Config(shape.num_layers, shape.hidden, shape.num_q_heads, shape.num_kv_heads,
                    shape.head_dim, shape.intermediate, shape.vocab,
                    int(shape.tie_embeddings), shape.rms_eps, shape.rope_theta)
        self._cfg = c

        def ptr(name):
            a = _req(weights[name], np.uint16)
            self._keep.append(a)
            return a.ctypes.data

        L = shape.num_layers
        layers = (_Layer * L)()
        for l in range(L):
            p = f"model.layers.{l}."
            layers[l] = _Layer(ptr(p + "input_layernorm.weight"),
                               ptr(p + "self_attn.q_proj.weight"),
                               ptr(p + "self_attn.k_proj.weight"),
                               ptr(p + "self_attn.v_proj.weight"),
                               ptr(p + "self_attn.o_proj.weight"),
                               ptr(p + "self_attn.q_norm.weight"),
                               ptr(p + "self_attn.k_norm.weight"),
                               ptr(p + "post_attention_layernorm.weight"),
                               ptr(p + "mlp.gate_proj.weight"),
                               ptr(p + "mlp.up_proj.weight"),
                               ptr(p + "mlp.down_proj.weight"))
        self._layers = layers
        lm = None if shape.tie_embeddings else ptr("lm_head.weight")
        self._w = _Weights(ptr("model.embed_tokens.weight"), ptr("model.norm.weight"), lm,
                           ctypes.cast(layers, ctypes.POINTER(_Layer)))

    def decode_step(self, tokens, positions, block_tables, pool: np.ndarray,
                    want_logits: bool = True, tap_layer: Optional[int] = None,
                    kv: KvFormat = BF16):
        """One decode step; appends to ``pool`` (of kv's type) in place.

        Returns (logits [B, V] float64 or None, next [B] int32, taps dict)."""
        lib = _load()
        s = self.shape
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        pool = _req(pool, kv.dtype)
        B = tokens.shape[0]
        assert positions.shape == (B,) and tables.shape[0] == B
        assert pool.shape[0] == s.num_layers and pool.shape[2] == 2
        logits = np.empty((B, s.vocab), dtype=np.float64) if want_logits else None
        nxt = np.empty(B, dtype=np.int32)
        taps = {}
        tp = None
        if tap_layer is not None:
            QD, KD = s.q_dim, s.kv_dim
            dims = {"x_in": (B, s.hidden), "qkv": (B, QD + 2 * KD),
                    "q_rot": (B, s.num_q_heads, s.head_dim),
                    "k_rot": (B, s.num_kv_heads, s.head_dim),
                    "attn": (B, s.num_q_heads, s.head_dim), "x_mid": (B, s.hidden),
                    "act": (B, s.intermediate), "x_out": (B, s.hidden),
                    "final_h": (B, s.hidden)}
            taps = {k: np.zeros(v, dtype=np.float64) for k, v in dims.items()}
            tp = _Taps(int(tap_layer), *[taps[n].ctypes.data for n in TAP_NAMES])
        rc = lib.or_decode_step(ctypes.byref(self._cfg), ctypes.byref(self._w), B,
                                tokens.ctypes.data, positions.ctypes.data, tables.ctypes.data,
                                tables.shape[1], pool.ctypes.data, pool.shape[1],
                                logits.ctypes.data if logits is not None else None,
                                nxt.ctypes.data, ctypes.byref(tp) if tp is not None else None,
                                ctypes.byref(kv._c()))
        if rc != 0:
            raise ValueError("oracle rejected the step arguments")
        return logits, nxt, taps

    def prefill(self, prompt, block_table_row, pool: np.ndarray, kv: KvFormat = BF16):
        """Run the prompt through the decoder one position at a time (0..T-1),
        filling the pool; returns (logits of the last position, greedy next id)."""
        prompt = np.asarray(prompt, dtype=np.int32)
        row = np.ascontiguousarray(np.asarray(block_table_row, dtype=np.int32)[None, :])
        logits = nxt = None
        for t in range(len(prompt)):
            logits, nxt, _ = self.decode_step(prompt[t:t + 1], np.array([t], np.int32), row,
                                              pool, want_logits=(t == len(prompt) - 1), kv=kv)
        return logits[0], int(nxt[0])

    def prefill_chunk(self, tokens, positions, block_tables, pool: np.ndarray, n_head: int,
                      kv: KvFormat = BF16):
        """The rows of a chunk through the layers as one batch, as
        ``decode_step`` runs its rows: per layer every row's K/V is appended at
        its position before any row attends, so rows of one sequence at
        consecutive positions get the causal prefill of that stretch (the blog
        "GPU 算子与执行优化：从 26 到 100 token/s", Part 7).  The steps are
        ``decode_step``'s; only the projections differ, as fp64 matrix
        products (numpy) of the bf16 weights, whose summation order is the
        library's, so the two agree to fp64 rounding.  Norms, RoPE, attention,
        SwiGLU and bf16 rounding are the C routines.  Only rows 0..n_head-1
        get the final norm, the LM head and the greedy id (the same Part 7:
        the LM head runs on the positions whose next token is wanted).
        Appends to ``pool`` in place; returns (logits [n_head, V], next
        [n_head])."""
        s = self.shape
        W = self._weights
        tokens = np.asarray(tokens, dtype=np.int32)
        positions = np.asarray(positions, dtype=np.int32)
        tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        pool = _req(pool, kv.dtype)
        B = tokens.shape[0]
        H, Hq, Hkv, D = s.hidden, s.num_q_heads, s.num_kv_heads, s.head_dim
        eps, theta = s.rms_eps, s.rope_theta
        assert positions.shape == (B,) and tables.shape[0] == B and 0 <= n_head <= B

        def mat(name):
            return bf16_to_f64(W[name])

        x = bf16_to_f64(W["model.embed_tokens.weight"][tokens])
        for l in range(s.num_layers):
            p = f"model.layers.{l}."
            h = rmsnorm(x, W[p + "input_layernorm.weight"], eps)
            q = (h @ mat(p + "self_attn.q_proj.weight").T).reshape(B, Hq, D)
            k = (h @ mat(p + "self_attn.k_proj.weight").T).reshape(B, Hkv, D)
            v = (h @ mat(p + "self_attn.v_proj.weight").T).reshape(B, Hkv, D)
            q = rmsnorm(q, W[p + "self_attn.q_norm.weight"], eps)
            k = rmsnorm(k, W[p + "self_attn.k_norm.weight"], eps)
            for b in range(B):
                q[b] = rope_neox(q[b], int(positions[b]), theta)
                k[b] = rope_neox(k[b], int(positions[b]), theta)
            if kv.fp8:
                kb, vb = f64_to_e4m3(k / kv.k_scale), f64_to_e4m3(v / kv.v_scale)
            else:
                kb, vb = f64_to_bf16(k), f64_to_bf16(v)
            for b in range(B):
                pos = int(positions[b])
                page = int(tables[b][pos // PAGE])
                if not 0 <= page < pool.shape[1]:
                    raise ValueError("block-table entry outside the pool")
                pool[l, page, 0, :, pos % PAGE, :] = kb[b]
                pool[l, page, 1, :, pos % PAGE, :] = vb[b]
            att = np.stack([attention(q[b], pool, l, tables[b], int(positions[b]) + 1, Hkv, kv)
                            for b in range(B)]).reshape(B, Hq * D)
            x = x + att @ mat(p + "self_attn.o_proj.weight").T
            h2 = rmsnorm(x, W[p + "post_attention_layernorm.weight"], eps)
            a = silu(h2 @ mat(p + "mlp.gate_proj.weight").T) * (h2 @ mat(p + "mlp.up_proj.weight").T)
            x = x + a @ mat(p + "mlp.down_proj.weight").T
        head = W["model.embed_tokens.weight"] if s.tie_embeddings else W["lm_head.weight"]
        hf = rmsnorm(x[:n_head], W["model.norm.weight"], eps)
        logits = linear(hf, head) if n_head else np.zeros((0, s.vocab))
        nxt = np.array([argmax(r) for r in logits], dtype=np.int32)
        return logits, nxt
